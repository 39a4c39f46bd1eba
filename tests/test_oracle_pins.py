"""Pins for the float64 oracle: each test ties it to something other than itself.

- brute force: explicit scalar loops on tiny ragged inputs (no numpy matmul);
- associativity: the absorbed order the MLA principle page gives (W_UK folded
  into the query, W_UV applied after P·c, its eqs. (4)-(5)) equals the oracle's
  original order (eqs. (1)-(2));
- library routines: torch's scaled_dot_product_attention and rms_norm in
  float64 on the CPU;
- RoPE: hand-evaluated textbook rotations, complex-number form, and the
  invariants of rotating only the rotary sub-dims;
- closed forms and consistency properties of causal softmax attention;
- page facts: the shape numbers the pages print (tests/golden/page_facts.json).
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O



GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_layer(rng, d_model, H, G, r, d_r, d_nope, d_v):
    return {
        "w_dkv": rng.standard_normal((r, d_model)) / math.sqrt(d_model),
        "w_kr": rng.standard_normal((G * d_r, d_model)) / math.sqrt(d_model),
        "w_qc": rng.standard_normal((H * d_nope, d_model)) / math.sqrt(d_model),
        "w_qr": rng.standard_normal((H * d_r, d_model)) / math.sqrt(d_model),
        "w_uk": rng.standard_normal((H, d_nope, r)) / math.sqrt(r),
        "w_uv": rng.standard_normal((H, d_v, r)) / math.sqrt(r),
    }


def _ragged(lengths):
    seg = np.concatenate([np.full(n, b) for b, n in enumerate(lengths)])
    pos = np.concatenate([np.arange(n) for n in lengths])
    return seg, pos


def _run(x, w, seg, pos, *, H, G, d_nope, d_r, theta, scale, norm=False, eps=1e-6):
    return O.mla_layer(x, x, w, k_pos=pos, q_pos=pos, k_seg=seg, q_seg=seg, n_heads=H,
                       n_groups=G, d_nope=d_nope, d_rope=d_r, theta=theta, scale=scale,
                       latent_rmsnorm=norm, eps=eps)


# ----------------------------------------------------------------------------
# P1: brute force with scalar loops
# ----------------------------------------------------------------------------


def _brute(x, w, seg, pos, *, H, G, d_nope, d_r, theta, scale, norm, eps):
    T, D = x.shape
    r = w["w_dkv"].shape[0]
    d_v = w["w_uv"].shape[1]
    half = d_r // 2

    def dot(a, b):
        s = 0.0
        for i in range(len(a)):
            s += float(a[i]) * float(b[i])
        return s

    def rot(vec, p):
        out = [0.0] * d_r
        for j in range(half):
            ang = p * theta ** (-2.0 * j / d_r)
            cs, sn = math.cos(ang), math.sin(ang)
            out[j] = vec[j] * cs - vec[j + half] * sn
            out[j + half] = vec[j + half] * cs + vec[j] * sn
        return out

    c = [[dot(x[t], w["w_dkv"][i]) for i in range(r)] for t in range(T)]
    if norm:
        for t in range(T):
            ms = sum(v * v for v in c[t]) / r
            c[t] = [v / math.sqrt(ms + eps) for v in c[t]]
    kr = [[rot([dot(x[t], w["w_kr"][g * d_r + j]) for j in range(d_r)], pos[t]) for g in range(G)]
          for t in range(T)]
    qn = [[[dot(x[t], w["w_qc"][h * d_nope + j]) for j in range(d_nope)] for h in range(H)]
          for t in range(T)]
    qr = [[rot([dot(x[t], w["w_qr"][h * d_r + j]) for j in range(d_r)], pos[t]) for h in range(H)]
          for t in range(T)]
    kn = [[[dot(w["w_uk"][h][j], c[s]) for j in range(d_nope)] for h in range(H)] for s in range(T)]
    v = [[[dot(w["w_uv"][h][j], c[s]) for j in range(d_v)] for h in range(H)] for s in range(T)]
    per = H // G
    out = np.zeros((T, H, d_v))
    for t in range(T):
        for h in range(H):
            keys = [s for s in range(T) if seg[s] == seg[t] and pos[s] <= pos[t]]
            logits = [scale * (dot(qn[t][h], kn[s][h]) + dot(qr[t][h], kr[s][h // per])) for s in keys]
            mx = max(logits)
            ex = [math.exp(a - mx) for a in logits]
            den = sum(ex)
            for e in range(d_v):
                out[t, h, e] = sum(ex[i] / den * v[keys[i]][h][e] for i in range(len(keys)))
    return out


@pytest.mark.parametrize("G,norm", [(1, False), (2, False), (2, True), (1, True)])
def test_p1_brute_force_ragged(G, norm):
    rng = np.random.default_rng(7 + G + 10 * norm)
    H, r, d_r, d_nope, d_v, D = 4, 6, 4, 3, 5, 8
    w = _rand_layer(rng, D, H, G, r, d_r, d_nope, d_v)
    lengths = [7, 4]
    seg, pos = _ragged(lengths)
    pos = pos + np.array([3] * 7 + [0] * 4)  # sequence 0 starts at position 3
    x = rng.standard_normal((sum(lengths), D))
    kw = dict(H=H, G=G, d_nope=d_nope, d_r=d_r, theta=10000.0, scale=0.37, norm=norm, eps=1e-6)
    got = _run(x, w, seg, pos, **kw)
    ref = _brute(x, w, seg, pos, **kw)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# P2: associativity — absorbed order equals the original order
# ----------------------------------------------------------------------------


def _absorbed(x, w, seg, pos, *, H, G, d_nope, d_r, theta, scale, norm=False, eps=1e-6):
    """Eqs. (4)-(5) of the MLA principle page, with W_UK absorbed into the query."""
    r = w["w_dkv"].shape[0]
    rows = O.cache_rows(x, w["w_dkv"], w["w_kr"], pos, n_groups=G, d_rope=d_r, theta=theta,
                        latent_rmsnorm=norm, eps=eps)
    c, kr = O.split_rows(rows, r, G, d_r)
    qn, qr = O.query(x, w["w_qc"], w["w_qr"], pos, n_heads=H, d_nope=d_nope, d_rope=d_r, theta=theta)
    q_lat = O.absorbed_query(qn, w["w_uk"])  # [T, H, r]: the function every q_lat check uses
    g = np.arange(H) // (H // G)
    s_lat = np.einsum("qhc,lc->hql", q_lat, c)
    s_pe = np.einsum("qhd,lhd->hql", qr, kr[:, g, :])
    a = scale * (s_lat + s_pe)
    allowed = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    a = np.where(allowed[None], a, -np.inf)
    p = np.exp(a - a.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    o_ = np.einsum("bhql,blc->bhqc", p[None], c[None])  # eq. (4)
    o = np.einsum("bhqc,hdc->bhqd", o_, w["w_uv"])       # eq. (5)
    return o[0].transpose(1, 0, 2)


@pytest.mark.parametrize("G", [1, 4])
def test_p2_associativity(G):
    rng = np.random.default_rng(11 + G)
    H, r, d_r, d_nope, d_v, D = 8, 24, 6, 5, 7, 16  # d_nope != r != d_v catches transposes
    w = _rand_layer(rng, D, H, G, r, d_r, d_nope, d_v)
    seg, pos = _ragged([9, 1, 5])
    x = rng.standard_normal((15, D))
    kw = dict(H=H, G=G, d_nope=d_nope, d_r=d_r, theta=500.0, scale=0.21)
    np.testing.assert_allclose(_run(x, w, seg, pos, **kw), _absorbed(x, w, seg, pos, **kw),
                               rtol=1e-11, atol=1e-12)


def test_absorbed_query_matches_page_einsum():
    rng = np.random.default_rng(3)
    qn = rng.standard_normal((5, 4, 3))
    w_uk = rng.standard_normal((4, 3, 7))
    ref = np.einsum("hdc,bhqd->bhqc", w_uk, qn.transpose(1, 0, 2)[None])[0].transpose(1, 0, 2)
    np.testing.assert_allclose(O.absorbed_query(qn, w_uk), ref, rtol=1e-13)


# ----------------------------------------------------------------------------
# P3: library routines in float64
# ----------------------------------------------------------------------------


def test_p3_sdpa_library_masked():
    rng = np.random.default_rng(5)
    Tq, S, H, d, e = 6, 9, 3, 8, 5
    q, k, v = rng.standard_normal((Tq, H, d)), rng.standard_normal((S, H, d)), rng.standard_normal((S, H, e))
    allowed = rng.random((Tq, S)) < 0.6
    allowed[:, 0] = True
    got = O.softmax_attention(q, k, v, allowed, 0.3)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(allowed), scale=0.3)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_p3_sdpa_is_causal_pins_mask_direction():
    """Single sequence, positions 0..n-1: the oracle's causal rule equals SDPA's is_causal."""
    rng = np.random.default_rng(8)
    H, r, d_r, d_nope, d_v, D, n = 2, 10, 4, 6, 3, 12, 11
    w = _rand_layer(rng, D, H, 1, r, d_r, d_nope, d_v)
    x = rng.standard_normal((n, D))
    pos, seg = np.arange(n), np.zeros(n, int)
    scale = 0.4
    got = _run(x, w, seg, pos, H=H, G=1, d_nope=d_nope, d_r=d_r, theta=10000.0, scale=scale)
    rows = O.cache_rows(x, w["w_dkv"], w["w_kr"], pos, n_groups=1, d_rope=d_r, theta=10000.0)
    c, kr = O.split_rows(rows, r, 1, d_r)
    qn, qr = O.query(x, w["w_qc"], w["w_qr"], pos, n_heads=H, d_nope=d_nope, d_rope=d_r, theta=10000.0)
    kn, v = O.expand_kv(c, w["w_uk"], w["w_uv"])
    Q = torch.from_numpy(np.concatenate([qn, qr], -1)).permute(1, 0, 2)[None]
    K = torch.from_numpy(np.concatenate([kn, np.repeat(kr, H, axis=1)], -1)).permute(1, 0, 2)[None]
    V = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_p3_rmsnorm_library():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((7, 33)) * 3.0
    ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (33,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(v, 1e-6), ref, rtol=1e-13)
    # closed form: ±a alternating has mean square a^2
    a = 2.5
    alt = np.array([a, -a] * 4)
    np.testing.assert_allclose(O.rmsnorm(alt, 1e-6), alt / math.sqrt(a * a + 1e-6), rtol=1e-15)


# ----------------------------------------------------------------------------
# P4: RoPE — textbook values and invariants
# ----------------------------------------------------------------------------


def test_p4_rope_hand_values():
    """d_r = 4, θ = 10000, p = 1: pairs (0,2) turn by 1 rad, pairs (1,3) by 10000^(-1/2) = 0.01 rad."""
    y = np.array([1.0, 2.0, 3.0, 4.0])
    got = O.rope(y, 1, 10000.0)
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    ref = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    np.testing.assert_allclose(got, ref, rtol=1e-15)


def test_p4_rope_complex_form():
    """Pair (y_j, y_{j+half}) as a complex number, multiplied by e^{i·p·θ_j}."""
    rng = np.random.default_rng(4)
    d, theta = 16, 10000.0
    y = rng.standard_normal(d)
    for p in [0, 1, 17, 4095, 131071]:
        got = O.rope(y, p, theta)
        for j in range(d // 2):
            z = complex(y[j], y[j + d // 2]) * cmath.exp(1j * p * theta ** (-2 * j / d))
            assert abs(got[j] - z.real) < 1e-12 and abs(got[j + d // 2] - z.imag) < 1e-12


def test_p4_rope_invariants():
    rng = np.random.default_rng(9)
    y = rng.standard_normal((5, 3, 8))
    # (a) p = 0 is the identity
    np.testing.assert_array_equal(O.rope(y, np.zeros(5), 10000.0), y)
    # (b) norm preserved
    yr = O.rope(y, np.arange(5) * 1000, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(yr, axis=-1), np.linalg.norm(y, axis=-1), rtol=1e-13)
    # (f) composition
    p1, p2 = np.array([3, 5, 7, 11, 13]), np.array([100, 0, 2, 9, 4096])
    np.testing.assert_allclose(O.rope(O.rope(y, p1, 10000.0), p2, 10000.0), O.rope(y, p1 + p2, 10000.0),
                               rtol=1e-11, atol=1e-12)


def _layer_parts(x, w, pos, H, G, d_nope, d_r, theta):
    r = w["w_dkv"].shape[0]
    rows = O.cache_rows(x, w["w_dkv"], w["w_kr"], pos, n_groups=G, d_rope=d_r, theta=theta)
    c, kr = O.split_rows(rows, r, G, d_r)
    qn, qr = O.query(x, w["w_qc"], w["w_qr"], pos, n_heads=H, d_nope=d_nope, d_rope=d_r, theta=theta)
    return c, kr, qn, qr


def test_p4_rotation_only_on_rotary_dims_and_relative():
    rng = np.random.default_rng(12)
    H, G, r, d_r, d_nope, d_v, D, n = 4, 2, 8, 6, 5, 3, 10, 6
    w = _rand_layer(rng, D, H, G, r, d_r, d_nope, d_v)
    x = rng.standard_normal((n, D))
    seg = np.zeros(n, int)
    kw = dict(H=H, G=G, d_nope=d_nope, d_r=d_r, theta=10000.0, scale=0.5)
    pos = np.arange(n)
    base = _run(x, w, seg, pos, **kw)
    # (c) shifting every position by Δ leaves the output unchanged (relative property)
    np.testing.assert_allclose(_run(x, w, seg, pos + 777, **kw), base, rtol=1e-10, atol=1e-12)
    # (e) positions change only the rotary parts: c and qn bit-identical, kr/qr not
    a = _layer_parts(x, w, pos, H, G, d_nope, d_r, 10000.0)
    b = _layer_parts(x, w, pos + 5, H, G, d_nope, d_r, 10000.0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[2], b[2])
    assert not np.allclose(a[1], b[1]) and not np.allclose(a[3], b[3])
    # (d) with W_QR = W_KR = 0 the output does not depend on positions at all
    w0 = dict(w, w_qr=np.zeros_like(w["w_qr"]), w_kr=np.zeros_like(w["w_kr"]))
    np.testing.assert_array_equal(_run(x, w0, seg, pos, **kw), _run(x, w0, seg, pos * 3 + 1, **kw))


# ----------------------------------------------------------------------------
# P5: closed forms
# ----------------------------------------------------------------------------


def test_p5_hand_example_quarter_three_quarters():
    """Hand-built layer: scores 0 and ln 3 give P = (1/4, 3/4) and o = (v0 + 3·v1)/4 = 5."""
    scale = 1.0 / math.sqrt(3.0)  # d_nope = 1, d_r = 2
    b = math.sqrt(3.0) * math.log(3.0)
    w = {
        "w_dkv": np.eye(2),                      # c0 = [1,0], c1 = [0,1]
        "w_kr": np.zeros((2, 2)),
        "w_qc": np.array([[0.0, 1.0]]),          # qn(token1) = 1, qn(token0) = 0
        "w_qr": np.zeros((2, 2)),
        "w_uk": np.array([[[0.0, b]]]),          # kn0 = 0, kn1 = b
        "w_uv": np.array([[[2.0, 6.0]]]),        # v0 = 2, v1 = 6
    }
    x = np.eye(2)
    out = _run(x, w, np.zeros(2, int), np.arange(2), H=1, G=1, d_nope=1, d_r=2, theta=10000.0,
               scale=scale)
    assert abs(out[0, 0, 0] - 2.0) < 1e-14          # token 0 sees only itself
    assert abs(out[1, 0, 0] - 5.0) < 1e-13


def test_p5_hand_example_rotary_cosine():
    """Only the rotary part scores: with d_r = 2 and θ_0 = 1, q·k = cos(p_q − p_k)."""
    w = {
        "w_dkv": np.eye(2), "w_kr": np.array([[1.0, 0.0], [0.0, 0.0]]),
        "w_qc": np.zeros((1, 2)), "w_qr": np.array([[1.0, 0.0], [0.0, 0.0]]),
        "w_uk": np.zeros((1, 1, 2)), "w_uv": np.array([[[1.0, -1.0]]]),
    }
    x = np.array([[1.0, 3.0], [1.0, 5.0]])  # c = x; v0 = -2, v1 = -4; rotary inputs [1, 0]
    scale = 0.8
    out = _run(x, w, np.zeros(2, int), np.arange(2), H=1, G=1, d_nope=1, d_r=2, theta=10000.0,
               scale=scale)
    e0, e1 = math.exp(scale * math.cos(1.0)), math.exp(scale * 1.0)
    assert abs(out[1, 0, 0] - (e0 * -2.0 + e1 * -4.0) / (e0 + e1)) < 1e-13


def test_p5_closed_forms():
    rng = np.random.default_rng(21)
    H, G, r, d_r, d_nope, d_v, D, n = 3, 1, 7, 4, 5, 6, 9, 8
    w = _rand_layer(rng, D, H, G, r, d_r, d_nope, d_v)
    x = rng.standard_normal((n, D))
    seg, pos = np.zeros(n, int), np.arange(n)
    kw = dict(H=H, G=G, d_nope=d_nope, d_r=d_r, theta=10000.0, scale=0.3)
    c = x @ w["w_dkv"].T
    v = np.einsum("hdc,sc->shd", w["w_uv"], c)
    # (a) first token attends only itself: o = v0
    out = _run(x, w, seg, pos, **kw)
    np.testing.assert_allclose(out[0], v[0], rtol=1e-13)
    # (b) zero queries: uniform weights, o = prefix mean of v
    wz = dict(w, w_qc=np.zeros_like(w["w_qc"]), w_qr=np.zeros_like(w["w_qr"]))
    outz = _run(x, wz, seg, pos, **kw)
    for t in range(n):
        np.testing.assert_allclose(outz[t], v[:t + 1].mean(axis=0), rtol=1e-12, atol=1e-14)
    # (c) all keys identical (same x at every position, no rotary): o = that v
    xs = np.repeat(x[:1], n, axis=0)
    w0 = dict(w, w_qr=np.zeros_like(w["w_qr"]), w_kr=np.zeros_like(w["w_kr"]))
    outs = _run(xs, w0, seg, pos, **kw)
    np.testing.assert_allclose(outs[-1], np.broadcast_to(v[0], outs[-1].shape), rtol=1e-12)
    # (d) a huge scale makes the top-scoring key dominate
    outd = _run(x, w, seg, pos, **dict(kw, scale=1e4))
    rows = O.cache_rows(x, w["w_dkv"], w["w_kr"], pos, n_groups=G, d_rope=d_r, theta=10000.0)
    cc, kr = O.split_rows(rows, r, G, d_r)
    qn, qr = O.query(x, w["w_qc"], w["w_qr"], pos, n_heads=H, d_nope=d_nope, d_rope=d_r, theta=10000.0)
    kn, _ = O.expand_kv(cc, w["w_uk"], w["w_uv"])
    t = n - 1
    for h in range(H):
        s = [qn[t, h] @ kn[j, h] + qr[t, h] @ kr[j, 0] for j in range(n)]
        np.testing.assert_allclose(outd[t, h], v[int(np.argmax(s)), h], rtol=1e-6, atol=1e-9)


# ----------------------------------------------------------------------------
# P6: consistency of the causal, segmented computation
# ----------------------------------------------------------------------------


def test_p6_consistency():
    rng = np.random.default_rng(31)
    H, G, r, d_r, d_nope, d_v, D = 4, 2, 8, 4, 3, 5, 12
    w = _rand_layer(rng, D, H, G, r, d_r, d_nope, d_v)
    kw = dict(H=H, G=G, d_nope=d_nope, d_r=d_r, theta=10000.0, scale=0.45)
    lengths = [6, 3, 8]
    seg, pos = _ragged(lengths)
    x = rng.standard_normal((sum(lengths), D))
    full = _run(x, w, seg, pos, **kw)
    # ragged batch == independent runs; decode of the last token == prefill row
    off = 0
    for b, n in enumerate(lengths):
        xb = x[off:off + n]
        one = _run(xb, w, np.zeros(n, int), np.arange(n), **kw)
        np.testing.assert_allclose(full[off:off + n], one, rtol=1e-12, atol=1e-14)
        dec = O.mla_layer(xb, xb[-1:], w, k_pos=np.arange(n), q_pos=np.array([n - 1]),
                          k_seg=np.zeros(n, int), q_seg=np.zeros(1, int), n_heads=H, n_groups=G,
                          d_nope=d_nope, d_rope=d_r, theta=10000.0, scale=0.45)
        np.testing.assert_allclose(dec[0], one[-1], rtol=1e-12, atol=1e-14)
        # prefix stability: a shorter prefix gives the same earlier rows
        pre = _run(xb[:n - 1], w, np.zeros(n - 1, int), np.arange(n - 1), **kw)
        np.testing.assert_allclose(pre, one[:n - 1], rtol=1e-12, atol=1e-14)
        off += n
    # permuting sequences permutes outputs
    order = [2, 0, 1]
    offs = np.cumsum([0] + lengths)
    xp = np.concatenate([x[offs[b]:offs[b + 1]] for b in order])
    segp, posp = _ragged([lengths[b] for b in order])
    outp = _run(xp, w, segp, posp, **kw)
    np.testing.assert_allclose(outp, np.concatenate([full[offs[b]:offs[b + 1]] for b in order]),
                               rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------
# P7: page facts fix the workload shapes
# ----------------------------------------------------------------------------


def test_p7_page_facts_and_workload_shapes():
    from mla_inputs import CONFIGS
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    f = lambda k: facts[k]["value"]  # noqa: E731
    # Qwen2.5-7B MLAfication: 4 KV heads x 128 x 2 = 1024 values -> 128 + 4x8 = 160, >= 6x smaller
    assert 4 * 128 * 2 == f("qwen25_gqa_kv_values_per_token")
    c2 = CONFIGS["qwen25_7b_decode"]
    assert c2.rank == f("qwen25_latent_rank") and c2.d_rope == f("qwen25_rope_dims_per_kv_head")
    assert c2.row_width == f("qwen25_mla_values_per_token")
    assert f("qwen25_gqa_kv_values_per_token") / c2.row_width >= f("qwen25_compression_at_least")
    # DeepSeek-V2: 24576 = H * (d_nope + d_r); o_proj input H * d_v = 16384; hidden 5120
    c3 = CONFIGS["deepseek_v2_decode"]
    assert c3.n_heads * (c3.d_nope + c3.d_rope) == f("deepseek_v2_q_b_proj_out")
    assert c3.n_heads * c3.d_v == f("deepseek_v2_o_proj_in")
    assert c3.d_model == f("deepseek_v2_hidden")
    from mla_inputs import Q_LORA_RANK
    assert Q_LORA_RANK == f("deepseek_v2_q_down_rank")  # the low-rank query's middle width
    # Qwen3-30B-A3B delta: rank 512, 8 rotary dims per KV head
    c4 = CONFIGS["qwen3_30b_ragged_decode"]
    assert c4.rank == f("qwen3_30b_latent_rank") and c4.d_rope == f("qwen3_30b_rope_dims_per_kv_head")
    # Zebra MLA layers: rank 256, hidden 2048, 16 heads
    c5 = CONFIGS["long_prefill_131k"]
    assert (c5.rank, c5.d_model, c5.n_heads) == (f("zebra_kv_lora_rank"), f("zebra_hidden"), f("zebra_heads"))
    nw = f("nanowhale_head_dim_split")
    assert nw["head_dim"] == nw["qk_rope_head_dim"] + nw["nope_head_dim"]


# ----------------------------------------------------------------------------
# P8: low-rank query path and output projection (beyond the attention)
# ----------------------------------------------------------------------------


def _lowrank_layer(rng, d_model, q_rank, H, d_nope, d_r, gain=True):
    return {
        "w_qa": rng.standard_normal((q_rank, d_model)) / math.sqrt(d_model),
        "q_gain": 1.0 + 0.1 * rng.standard_normal(q_rank) if gain else None,
        "w_qb": rng.standard_normal((H * (d_nope + d_r), q_rank)) / math.sqrt(q_rank),
    }


def test_p8_lowrank_query_brute_force():
    """Scalar loops: down-projection, RMSNorm with gain, up-projection, per-head
    split [q_nope ; q_pe] (no-position part first), then the rotation of q_pe
    (d_r = 2: the single pair turns by p radians)."""
    rng = np.random.default_rng(80)
    d_model, q_rank, H, d_nope, d_r, eps = 6, 4, 2, 3, 2, 1e-6
    w = _lowrank_layer(rng, d_model, q_rank, H, d_nope, d_r)
    x = rng.standard_normal((3, d_model))
    pos = np.array([0, 1, 5])
    qn, qr = O.lowrank_query(x, w["w_qa"], w["q_gain"], w["w_qb"], pos, n_heads=H, d_nope=d_nope,
                             d_rope=d_r, theta=10000.0, eps=eps)
    for t in range(3):
        cq = [sum(x[t][k] * w["w_qa"][i][k] for k in range(d_model)) for i in range(q_rank)]
        ms = sum(v * v for v in cq) / q_rank
        cqn = [cq[i] / math.sqrt(ms + eps) * w["q_gain"][i] for i in range(q_rank)]
        q = [sum(cqn[i] * w["w_qb"][j][i] for i in range(q_rank)) for j in range(H * (d_nope + d_r))]
        for h in range(H):
            base = h * (d_nope + d_r)
            for d in range(d_nope):
                assert abs(qn[t, h, d] - q[base + d]) < 1e-12
            y0, y1 = q[base + d_nope], q[base + d_nope + 1]
            a = float(pos[t])
            assert abs(qr[t, h, 0] - (y0 * math.cos(a) - y1 * math.sin(a))) < 1e-12
            assert abs(qr[t, h, 1] - (y1 * math.cos(a) + y0 * math.sin(a))) < 1e-12


def test_p8_lowrank_query_library_and_invariants():
    """torch's float64 rms_norm with weight, then the linear maps; RMSNorm makes the
    query invariant to the scale of x (eps = 0); with q_rank = d_model, W_QA = I,
    unit gain and eps = 0 the path is the full-rank query of rmsnorm(x) whose
    W_QC / W_QR are W_QB's per-head no-position / rotary rows."""
    rng = np.random.default_rng(81)
    d_model, q_rank, H, d_nope, d_r = 12, 8, 3, 4, 4
    w = _lowrank_layer(rng, d_model, q_rank, H, d_nope, d_r)
    x = rng.standard_normal((5, d_model))
    pos = np.zeros(5, int)
    qn, qr = O.lowrank_query(x, w["w_qa"], w["q_gain"], w["w_qb"], pos, n_heads=H, d_nope=d_nope,
                             d_rope=d_r, theta=10000.0, eps=1e-6)
    tx = torch.from_numpy(x)
    cq = torch.nn.functional.rms_norm(tx @ torch.from_numpy(w["w_qa"]).T, (q_rank,),
                                      weight=torch.from_numpy(w["q_gain"]), eps=1e-6)
    q = (cq @ torch.from_numpy(w["w_qb"]).T).view(5, H, d_nope + d_r).numpy()
    np.testing.assert_allclose(qn, q[..., :d_nope], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(qr, q[..., d_nope:], rtol=1e-12, atol=1e-14)   # p = 0: no rotation
    pos = np.array([0, 3, 17, 100, 4095])
    a = O.lowrank_query(x, w["w_qa"], w["q_gain"], w["w_qb"], pos, n_heads=H, d_nope=d_nope, d_rope=d_r,
                        theta=10000.0, eps=0.0)
    b = O.lowrank_query(7.3 * x, w["w_qa"], w["q_gain"], w["w_qb"], pos, n_heads=H, d_nope=d_nope,
                        d_rope=d_r, theta=10000.0, eps=0.0)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)
    # reduction to the full-rank query
    wf = _lowrank_layer(rng, d_model, d_model, H, d_nope, d_r, gain=False)
    wf["w_qa"] = np.eye(d_model)
    qn_l, qr_l = O.lowrank_query(x, wf["w_qa"], None, wf["w_qb"], pos, n_heads=H, d_nope=d_nope,
                                 d_rope=d_r, theta=10000.0, eps=0.0)
    rows = wf["w_qb"].reshape(H, d_nope + d_r, d_model)
    w_qc = rows[:, :d_nope].reshape(H * d_nope, d_model)
    w_qr = rows[:, d_nope:].reshape(H * d_r, d_model)
    qn_f, qr_f = O.query(O.rmsnorm(x, 0.0), w_qc, w_qr, pos, n_heads=H, d_nope=d_nope, d_rope=d_r,
                         theta=10000.0)
    np.testing.assert_allclose(qn_l, qn_f, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(qr_l, qr_f, rtol=1e-12, atol=1e-14)


def test_p8_output_projection_brute_and_page_chain():
    """Scalar loops of u[D] = Σ_h Σ_e o[h,e]·W_o[D, h·d_v + e]; and the page's combined
    form of eqs. (1)-(3), einsum('hdc,blc,bqhl,hdD->bhD', W_UV, c, P, W_o), with P the
    softmax of explicit scores, equals output_projection(mla_attention(...))."""
    rng = np.random.default_rng(82)
    T, H, d_v, D = 3, 2, 3, 5
    o = rng.standard_normal((T, H, d_v))
    w_o = rng.standard_normal((D, H * d_v))
    u = O.output_projection(o, w_o)
    for t in range(T):
        for dd in range(D):
            ref = sum(o[t][h][e] * w_o[dd][h * d_v + e] for h in range(H) for e in range(d_v))
            assert abs(u[t, dd] - ref) < 1e-12
    # combined page form for the last query of one causal sequence
    d_model, r, d_r, d_nope, G, L = 10, 6, 4, 3, 1, 7
    w = _rand_layer(rng, d_model, H, G, r, d_r, d_nope, d_v)
    x = rng.standard_normal((L, d_model))
    seg, pos = _ragged([L])
    scale = 1.0 / math.sqrt(d_nope + d_r)
    o_all = _run(x, w, seg, pos, H=H, G=G, d_nope=d_nope, d_r=d_r, theta=10000.0, scale=scale)
    u_or = O.output_projection(o_all, w_o)[-1]
    c = x @ w["w_dkv"].T
    kn = np.einsum("hdc,lc->lhd", w["w_uk"], c)
    kr = O.rope((x @ w["w_kr"].T).reshape(L, G, d_r), pos, 10000.0)
    qn = (x[-1] @ w["w_qc"].T).reshape(H, d_nope)
    qr = O.rope((x[-1] @ w["w_qr"].T).reshape(1, H, d_r), pos[-1:], 10000.0)[0]
    s = scale * (np.einsum("hd,lhd->hl", qn, kn) + np.einsum("hd,ld->hl", qr, kr[:, 0]))
    P = np.exp(s - s.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    u_page = np.einsum("hdc,lc,hl,hdD->D", w["w_uv"], c, P, w_o.T.reshape(H, d_v, D))
    np.testing.assert_allclose(u_or, u_page, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# P9: the DeepSeek-V4 / nanowhale variant
# ----------------------------------------------------------------------------


def test_p9_rope_interleaved_complex_form_and_inverse():
    """Pairs (2j, 2j+1) times e^{i p f_j} (cmath), p = 0 identity, rotation by -p
    undoes p, and a given frequency table equal to θ^(-2j/d) gives the same result."""
    rng = np.random.default_rng(90)
    y = rng.standard_normal(8)
    p = 37.0
    got = O.rope_interleaved(y, p, 10000.0)
    for j in range(4):
        z = complex(y[2 * j], y[2 * j + 1]) * cmath.exp(1j * p * 10000.0 ** (-2.0 * j / 8))
        assert abs(got[2 * j] - z.real) < 1e-12 and abs(got[2 * j + 1] - z.imag) < 1e-12
    np.testing.assert_allclose(O.rope_interleaved(y, 0.0), y, rtol=0, atol=0)
    np.testing.assert_allclose(O.rope_interleaved(got, -p), y, rtol=1e-12, atol=1e-12)
    table = 10000.0 ** (-2.0 * np.arange(4) / 8)
    np.testing.assert_allclose(O.rope_interleaved(y, p, inv_freq=table), got, rtol=1e-14, atol=1e-14)


def _v4_small(rng, T=5, D=6, dr=2, H=2):
    q = rng.standard_normal((T, H, D))
    kv = rng.standard_normal((T, D))
    return q, kv


def test_p9_v4_attention_brute_force_and_library():
    """Scalar loops (sink in the denominator, K = V = the row, inverse rotation of
    the output's rotary pair by the query position); with sink = -inf the
    no-position dims equal torch's float64 SDPA of the expanded single head."""
    rng = np.random.default_rng(91)
    T, D, dr, H = 5, 6, 2, 2
    q, kv = _v4_small(rng, T, D, dr, H)
    sink = np.array([0.3, -1.2])
    pos = np.arange(T)
    seg = np.zeros(T, int)
    scale = 0.7
    got = O.v4_attention(q, kv, sink, pos, pos, seg, seg, scale, d_rope=dr)
    for t in range(T):
        for h in range(H):
            s = [scale * sum(q[t, h, d] * kv[u, d] for d in range(D)) for u in range(t + 1)]
            m = max(max(s), sink[h])
            e = [math.exp(v - m) for v in s]
            den = sum(e) + math.exp(sink[h] - m)
            o = [sum(e[u] * kv[u, d] for u in range(t + 1)) / den for d in range(D)]
            z = complex(o[D - 2], o[D - 1]) * cmath.exp(-1j * t * 1.0)   # f_0 = 1 for the single pair
            ref = o[:D - 2] + [z.real, z.imag]
            for d in range(D):
                assert abs(got[t, h, d] - ref[d]) < 1e-12
    no_sink = O.v4_attention(q, kv, np.full(H, -np.inf), pos, pos, seg, seg, scale, d_rope=dr)
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]
    K = torch.from_numpy(np.repeat(kv[:, None], H, 1)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, K, is_causal=True, scale=scale)[0]
    np.testing.assert_allclose(no_sink[..., :D - dr], ref.permute(1, 0, 2).numpy()[..., :D - dr],
                               rtol=1e-12, atol=1e-13)


def test_p9_v4_attention_closed_form_and_relative_positions():
    """One key: o = kv_0·e^s / (e^s + e^sink) on the no-position dims.  Rotating q and
    kv by their positions, then the output back by the query's, makes the output
    depend on relative positions only: shifting every position changes nothing."""
    rng = np.random.default_rng(92)
    D, dr, H = 8, 4, 3
    q = rng.standard_normal((1, H, D))
    kv = rng.standard_normal((1, D))
    sink = rng.standard_normal(H)
    o = O.v4_attention(q, kv, sink, [0], [0], [0], [0], 0.5, d_rope=dr)
    for h in range(H):
        s = 0.5 * float(q[0, h] @ kv[0])
        w = math.exp(s) / (math.exp(s) + math.exp(sink[h]))
        np.testing.assert_allclose(o[0, h, :D - dr], w * kv[0, :D - dr], rtol=1e-13)
    # relative positions: rows built from position-free parts, rotated at p and p + 1000
    T = 6
    qa = rng.standard_normal((T, H, D))
    ka = rng.standard_normal((T, D))
    seg = np.zeros(T, int)
    outs = []
    for shift in (0, 1000):
        pos = np.arange(T) + shift
        qq, kk = qa.copy(), ka.copy()
        qq[..., -dr:] = O.rope_interleaved(qa[..., -dr:], pos[:, None], 10000.0)
        kk[:, -dr:] = O.rope_interleaved(ka[:, -dr:], pos, 10000.0)
        outs.append(O.v4_attention(qq, kk, sink, pos, pos, seg, seg, 0.4, d_rope=dr))
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-9, atol=1e-11)


def test_p9_v4_projections_brute_force():
    """Cache rows (RMSNorm with gain, rotary tail), queries (low-rank, per-head rotary
    tail) and the grouped output projection against scalar loops; one output group
    is two plain products."""
    rng = np.random.default_rng(93)
    d_model, D, dr, H, qr, G, R = 5, 4, 2, 2, 3, 2, 3
    x = rng.standard_normal((3, d_model))
    pos = np.array([0, 2, 9])
    w_kv = rng.standard_normal((D, d_model))
    g_kv = 1 + 0.1 * rng.standard_normal(D)
    rows = O.v4_cache_rows(x, w_kv, g_kv, pos, d_rope=dr, eps=1e-6)
    for t in range(3):
        v = [sum(x[t, k] * w_kv[i, k] for k in range(d_model)) for i in range(D)]
        inv = 1 / math.sqrt(sum(a * a for a in v) / D + 1e-6)
        v = [v[i] * inv * g_kv[i] for i in range(D)]
        z = complex(v[2], v[3]) * cmath.exp(1j * pos[t])
        ref = v[:2] + [z.real, z.imag]
        np.testing.assert_allclose(rows[t], ref, rtol=1e-12, atol=1e-13)
    w_qa = rng.standard_normal((qr, d_model))
    g_q = 1 + 0.1 * rng.standard_normal(qr)
    w_qb = rng.standard_normal((H * D, qr))
    q = O.v4_query(x, w_qa, g_q, w_qb, pos, n_heads=H, head_dim=D, d_rope=dr, eps=1e-6)
    for t in range(3):
        c = [sum(x[t, k] * w_qa[i, k] for k in range(d_model)) for i in range(qr)]
        inv = 1 / math.sqrt(sum(a * a for a in c) / qr + 1e-6)
        c = [c[i] * inv * g_q[i] for i in range(qr)]
        for h in range(H):
            v = [sum(c[i] * w_qb[h * D + d, i] for i in range(qr)) for d in range(D)]
            z = complex(v[2], v[3]) * cmath.exp(1j * pos[t])
            np.testing.assert_allclose(q[t, h], v[:2] + [z.real, z.imag], rtol=1e-12, atol=1e-13)
    o = rng.standard_normal((3, H, D))
    gdim = H * D // G
    w_oa = rng.standard_normal((G * R, gdim))
    w_ob = rng.standard_normal((d_model, G * R))
    u = O.v4_output(o, w_oa, w_ob, G)
    flat = o.reshape(3, -1)
    for t in range(3):
        a = [sum(flat[t, g * gdim + d] * w_oa[g * R + r, d] for d in range(gdim)) for g in range(G) for r in range(R)]
        for j in range(d_model):
            assert abs(u[t, j] - sum(a[i] * w_ob[j, i] for i in range(G * R))) < 1e-11
    w1 = rng.standard_normal((R, H * D))
    np.testing.assert_allclose(O.v4_output(o, w1, w_ob[:, :R], 1), (flat @ w1.T) @ w_ob[:, :R].T, rtol=1e-12)


# ----------------------------------------------------------------------------
# P10: YaRN-rescaled rotary frequencies (Zebra hybrid page: factor 32 over a 32K
# window; the interpolation itself from the YaRN paper)
# ----------------------------------------------------------------------------


def test_p10_yarn_table_ends_and_midpoint():
    """θ = 16, d_rope = 8 gives θ_j = 2^-j; a window of 2π·16 turns pair j 16·2^-j
    times over it.  With the ramp on [4, 12]: pair 0 (16 turns) keeps its
    frequency, pair 3 (2 turns) is divided by the factor, and pair 1 (8 turns, the
    ramp's midpoint) gets the mean of the two."""
    s = 5.0
    f = O.yarn_inv_freq(8, 16.0, s, 2 * math.pi * 16, alpha=4.0, beta=12.0)
    assert f[0] == 1.0
    assert abs(f[3] - 0.125 / s) < 1e-16
    assert abs(f[1] - 0.5 * (0.5 / s + 0.5)) < 1e-15
    # factor 1 changes nothing, at the pages' shape (64 rotary dims, 32K window)
    plain = 10000.0 ** (-2.0 * np.arange(32) / 64)
    np.testing.assert_allclose(O.yarn_inv_freq(64, 10000.0, 1.0, 32768.0), plain, rtol=1e-15, atol=0)


def test_p10_yarn_table_bounds_and_order():
    """Every rescaled frequency lies in [θ_j/s, θ_j] and they fall with j; at the
    Zebra page's factor 32 over 32768 tokens the fastest pair is untouched and the
    slowest (fewer than one turn over the window) is interpolated fully."""
    s = 32.0
    f = O.yarn_inv_freq(64, 10000.0, s, 32768.0)
    plain = 10000.0 ** (-2.0 * np.arange(32) / 64)
    assert np.all(f <= plain * (1 + 1e-15)) and np.all(f >= plain / s * (1 - 1e-15))
    assert np.all(np.diff(f) < 0)
    assert f[0] == plain[0]
    assert abs(f[-1] - plain[-1] / s) < 1e-18
    assert np.any((f > plain / s * 1.01) & (f < plain * 0.99))    # some pairs on the ramp


def test_p10_yarn_interpolated_pairs_stretch_positions():
    """On the fully interpolated pairs, position s·p with the YaRN table turns exactly
    as p did with the original frequencies; on the untouched pairs nothing changes."""
    d, s, W = 64, 32.0, 32768.0
    f = O.yarn_inv_freq(d, 10000.0, s, W)
    plain = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    slow = np.isclose(f, plain / s, rtol=1e-14, atol=0)
    fast = f == plain
    assert slow.sum() >= 2 and fast.sum() >= 2
    rng = np.random.default_rng(100)
    y = rng.standard_normal(d)
    p = 1234.0
    got = O.rope(y, s * p, 10000.0, inv_freq=f)
    ref = O.rope(y, p, 10000.0)
    idx = np.nonzero(slow)[0]
    np.testing.assert_allclose(got[idx], ref[idx], rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(got[idx + d // 2], ref[idx + d // 2], rtol=1e-9, atol=1e-9)
    same = O.rope(y, p, 10000.0, inv_freq=f)
    jdx = np.nonzero(fast)[0]
    np.testing.assert_allclose(same[jdx], ref[jdx], rtol=0, atol=1e-15)


def test_p10_table_rope_keeps_rotation_properties():
    """With any frequency table the rotation keeps the norm and scores depend only on
    relative positions; the default table reproduces the untabled rotation."""
    rng = np.random.default_rng(101)
    d = 16
    f = O.yarn_inv_freq(d, 10000.0, 32.0, 4096.0)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    a = O.rope(q, 1_000_000.0, 10000.0, inv_freq=f) @ O.rope(k, 999_000.0, 10000.0, inv_freq=f)
    b = O.rope(q, 1000.0, 10000.0, inv_freq=f) @ O.rope(k, 0.0, 10000.0, inv_freq=f)
    assert abs(a - b) < 1e-9
    assert abs(np.linalg.norm(O.rope(q, 777.0, 10000.0, inv_freq=f)) - np.linalg.norm(q)) < 1e-12
    plain = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    np.testing.assert_allclose(O.rope(q, 77.0, 10000.0, inv_freq=plain), O.rope(q, 77.0, 10000.0),
                               rtol=0, atol=1e-15)


def test_p10_yarn_logit_scale():
    """The temperature's closed forms: factor 1 leaves the logits; factor e^10 gives
    √(1/t) = 2, so logits are multiplied by 4."""
    assert O.yarn_logit_scale(1.0) == 1.0
    assert abs(O.yarn_logit_scale(math.exp(10.0)) - 4.0) < 1e-12


# ----------------------------------------------------------------------------
# P11: the parity metric and the test harness's absorbed reference
# ----------------------------------------------------------------------------
# Every GPU parity claim is a value of O.max_rel_err compared with a bar, so the
# metric itself is pinned here on hand-built arrays whose answer is worked out by
# hand: per (token, head), ‖got − ref‖∞ / ‖ref‖∞ over the last axis, then the max.


def test_p11_max_rel_err_hand_values():
    ref = np.zeros((2, 3, 4))
    got = np.zeros((2, 3, 4))
    # (0, 0): a large reference; an error of 1 in a zero element gives 1/100
    ref[0, 0] = [100.0, 0.0, 0.0, 0.0]
    got[0, 0] = [100.0, 1.0, 0.0, 0.0]
    # (1, 2): a small reference; an error of 0.01 gives 0.01 / 0.1 = 0.1 (the max)
    ref[1, 2] = [0.1, -0.1, 0.1, 0.05]
    got[1, 2] = [0.1, -0.11, 0.1, 0.05]
    # (0, 1): ratio 0.5 / 20 = 0.025
    ref[0, 1] = [-20.0, 3.0, 0.0, 1.0]
    got[0, 1] = [-20.0, 3.0, 0.5, 1.0]
    # the remaining rows are all-zero references with exact results
    assert abs(O.max_rel_err(got, ref) - 0.1) < 1e-15
    # the mean over the rows would be (0.01 + 0.1 + 0.025) / 6, a global
    # normalisation 0.01 / 100, a per-element ratio infinite: none is 0.1
    assert O.max_rel_err(got[0], ref[0]) == pytest.approx(0.025, abs=1e-15)
    assert O.max_rel_err(got[0, 0], ref[0, 0]) == pytest.approx(0.01, abs=1e-15)


def test_p11_max_rel_err_axis_and_scale():
    """Normalised along the last axis only: transposing the two leading axes keeps the
    value, transposing the last one changes it; a common positive factor cancels."""
    ref = np.array([[[4.0, 0.0], [0.0, 0.5]]])       # rows (0,0) = [4, 0], (0,1) = [0, 0.5]
    got = np.array([[[4.0, 0.2], [0.0, 0.5]]])       # row (0,0): 0.2 / 4 = 0.05
    assert O.max_rel_err(got, ref) == pytest.approx(0.05, abs=1e-15)
    # along the other axis the rows would be [4, 0] / [0, 0.5]: 0 and 0.2 / 0.5 = 0.4
    assert O.max_rel_err(got.swapaxes(1, 2), ref.swapaxes(1, 2)) == pytest.approx(0.4, abs=1e-15)
    assert O.max_rel_err(got.swapaxes(0, 1), ref.swapaxes(0, 1)) == pytest.approx(0.05, abs=1e-15)
    assert O.max_rel_err(3.5 * got, 3.5 * ref) == pytest.approx(0.05, abs=1e-15)


def test_p11_max_rel_err_zero_reference_and_edges():
    """A row whose reference is all zero is measured by its absolute error; an empty
    input has no error; a NaN or inf in the result never passes a bar."""
    ref = np.array([[0.0, 0.0, 0.0], [1.0, 2.0, -2.0]])
    assert O.max_rel_err(np.array([[0.0, 0.0, 0.0], [1.0, 2.0, -2.0]]), ref) == 0.0
    assert O.max_rel_err(np.array([[0.0, 0.003, -0.004], [1.0, 2.0, -2.0]]), ref) == pytest.approx(0.004)
    assert O.max_rel_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    for bad in (np.nan, np.inf, -np.inf):
        got = ref.copy()
        got[1, 1] = bad
        e = O.max_rel_err(got, ref)
        assert not (e <= 1e-2), bad


def test_p11_harness_checker_is_the_oracle_metric():
    """The GPU tests' checker is the oracle's metric, not a second copy of it."""
    from tests import harness as Hh
    assert Hh.rel_err_rows is O.max_rel_err


@pytest.mark.parametrize("G", [1, 4])
def test_p11_harness_absorbed_reference_matches_expanded_oracle(G):
    """tests/harness.oracle_absorbed_rows (the reference of the restart tests: the
    query the kernels read, K = [c ; kr], V = c, then W_UV) equals the oracle's
    non-absorbed decode output when it is given the float64 absorbed query
    q_lat = O.absorbed_query(q_nope, W_UK) (associativity, eqs. (4)-(5))."""
    import types

    from tests import harness as Hh
    rng = np.random.default_rng(40 + G)
    H, r, d_r, d_nope, d_v, D, n = 8, 24, 6, 5, 7, 16, 13
    w = _rand_layer(rng, D, H, G, r, d_r, d_nope, d_v)
    cfg = types.SimpleNamespace(n_heads=H, rank=r, n_groups=G, d_rope=d_r, d_v=d_v, softmax_scale=0.29)
    x = rng.standard_normal((n, D))
    pos = np.arange(n) + 5
    rows = O.cache_rows(x, w["w_dkv"], w["w_kr"], pos, n_groups=G, d_rope=d_r, theta=700.0)
    qn, qr = O.query(x[-1:], w["w_qc"], w["w_qr"], pos[-1:], n_heads=H, d_nope=d_nope, d_rope=d_r,
                     theta=700.0)
    q_lat = O.absorbed_query(qn, w["w_uk"])[0]
    got = Hh.oracle_absorbed_rows(cfg, w, q_lat, qr[0], rows, head_chunk=3)
    c, kr = O.split_rows(rows, r, G, d_r)
    ref = O.mla_attention(qn, qr, c, kr, w["w_uk"], w["w_uv"], pos[-1:], pos, np.zeros(1, int),
                          np.zeros(n, int), 0.29)[0]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
