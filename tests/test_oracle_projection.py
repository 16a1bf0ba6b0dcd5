"""Pins of the per-head projection oracle (oracle/projection.py): brute force,
the identity map, and the two MLA identities it exists for (absorbing the key
up-projection into the query, and applying the value up-projection after
attention over the latent)."""
import math

import numpy as np

import oracle


def test_bruteforce_small():
    rng = np.random.default_rng(0)
    M, H, K, N = 3, 2, 5, 4
    x = rng.standard_normal((M, H, K))
    w = rng.standard_normal((H, K, N))
    y = oracle.head_project(x, w)
    for m in range(M):
        for h in range(H):
            for n in range(N):
                assert abs(y[m, h, n] - math.fsum(x[m, h, k] * w[h, k, n] for k in range(K))) < 1e-12


def test_identity_weights():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 3, 16))
    w = np.broadcast_to(np.eye(16), (3, 16, 16)).copy()
    assert np.array_equal(oracle.head_project(x, w), x)


def test_heads_are_independent():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 4, 8))
    w = rng.standard_normal((4, 8, 6))
    perm = np.array([2, 0, 3, 1])
    assert np.allclose(oracle.head_project(x[:, perm], w[perm]), oracle.head_project(x, w)[:, perm],
                       rtol=0, atol=1e-12)


def test_query_absorption_preserves_scores():
    """q_nope . (per-head key from the latent) == (q_nope absorbed) . latent."""
    rng = np.random.default_rng(3)
    M, H, dn, dl, P = 4, 3, 128, 512, 10
    q_nope = rng.standard_normal((M, H, dn))
    w_uk = rng.standard_normal((H, dn, dl)) / math.sqrt(dl)
    c_kv = rng.standard_normal((P, dl))
    q_lat = oracle.head_project(q_nope, w_uk)
    for h in range(H):
        k_nope = c_kv @ w_uk[h].T  # [P, dn]: each head's keys up-projected from the latent
        assert np.allclose(q_nope[:, h] @ k_nope.T, q_lat[:, h] @ c_kv.T, rtol=1e-10, atol=1e-10)


def test_value_projection_after_attention():
    """Projecting the latent output equals attending over per-head value rows."""
    rng = np.random.default_rng(4)
    H, P = 3, 12
    q_lat = rng.standard_normal((H, 512))
    q_rope = rng.standard_normal((H, 64))
    c_kv = rng.standard_normal((P, 512))
    k_rope = rng.standard_normal((P, 64))
    w_uv = rng.standard_normal((H, 512, 128)) / math.sqrt(512)
    scale = 1 / math.sqrt(192)
    out_lat, _ = oracle.attend(q_lat, q_rope, c_kv, k_rope, scale)  # [H, 512]
    o = oracle.head_project(out_lat[None], w_uv)[0]                  # [H, 128]
    s = scale * (q_lat @ c_kv.T + q_rope @ k_rope.T)
    a = np.exp(s - s.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)
    for h in range(H):
        v_h = c_kv @ w_uv[h]  # [P, 128]: this head's value rows
        assert np.allclose(a[h] @ v_h, o[h], rtol=1e-10, atol=1e-12)
