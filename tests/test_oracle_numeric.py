"""Pins of the oracle's numeric building blocks against closed forms,
invariants and independent library routines (PyTorch CPU, float64)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import fpd_oracle as O


# --- bfloat16 rounding -------------------------------------------------------

def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32),
        (rng.standard_normal(10_000) * 1e-30).astype(np.float32),
        (rng.standard_normal(10_000) * 1e30).astype(np.float32),
        np.float32([0.0, -0.0, 1.0, -1.0]),
    ])
    # exact ties: bf16 values plus half an ulp
    base = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16)
    bits = base.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
    ties = (bits | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_round_hand_values():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert O.bf16_round(1 + 2.0 ** -8) == 1.0
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert O.bf16_round(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    # just below 2 rounds up into the next binade
    assert O.bf16_round(2 - 2.0 ** -10) == 2.0
    assert O.bf16_round(-(1 + 2.0 ** -7)) == -(1 + 2.0 ** -7)
    # a float64 value just above a tie rounds up (no double rounding through float32)
    assert O.bf16_round(1 + 2.0 ** -8 + 2.0 ** -40) == 1 + 2.0 ** -7


# --- RMSNorm -----------------------------------------------------------------

def test_rmsnorm_matches_torch_and_has_unit_rms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 96)) * 3.0
    g = rng.standard_normal(96)
    got = O.rmsnorm(x, g, 1e-6)
    want = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    unit = O.rmsnorm(x, np.ones(96), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(unit ** 2, axis=-1)), 1.0, rtol=1e-12)


def test_rmsnorm_constant_input():
    # a constant row c maps to c / sqrt(c^2 + eps) * g
    out = O.rmsnorm(np.full((1, 8), -2.5), np.arange(8.0), 0.0)
    np.testing.assert_allclose(out, -np.arange(8.0)[None, :], rtol=1e-14)


# --- RoPE --------------------------------------------------------------------

def _rope_complex(x, pos, theta):
    """Rotate-half RoPE written as a complex product (x_i + j x_{i+d/2}) e^{j pos w_i}."""
    d = x.shape[-1]
    half = d // 2
    w = theta ** (-(np.arange(half) * 2.0) / d)
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * pos[:, None, None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("d", [64, 128])
def test_rope_equals_complex_rotation(d):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((11, 3, d))
    pos = np.arange(100, 111)
    np.testing.assert_allclose(O.rope(x, pos, 1e6), _rope_complex(x, pos, 1e6), atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    d = 128
    q = rng.standard_normal((5, 1, d))
    k = rng.standard_normal((5, 1, d))
    pq, pk = np.array([3, 9, 40, 4000, 77]), np.array([0, 1, 2, 3, 4000])
    r = O.rope(q, pq, 1e6)
    # per-pair norms are preserved
    np.testing.assert_allclose(r[..., :64] ** 2 + r[..., 64:] ** 2, q[..., :64] ** 2 + q[..., 64:] ** 2,
                               rtol=1e-12)
    # q_m . k_n depends only on m - n
    s1 = np.einsum("tid,tid->t", O.rope(q, pq, 1e6), O.rope(k, pk, 1e6))
    s2 = np.einsum("tid,tid->t", O.rope(q, pq + 517, 1e6), O.rope(k, pk + 517, 1e6))
    np.testing.assert_allclose(s1, s2, rtol=1e-9, atol=1e-9)
    # position 0 is the identity
    np.testing.assert_allclose(O.rope(q, np.zeros(5), 1e6), q, atol=0)


# --- attention ---------------------------------------------------------------

class _Shape:
    def __init__(self, **kw):
        d = dict(hidden=64, n_q=4, n_kv=2, head_dim=16, n_layers=1, inter=32, vocab=64, n_fused=1,
                 dtype="f32", rope_theta=1e6, use_rope=1, rms_eps=1e-6)
        d.update(kw)
        self.__dict__.update(d)


class _W:
    layers = []


@pytest.mark.parametrize("nq,nkv", [(4, 2), (8, 2), (4, 4), (6, 1)])
def test_attention_matches_torch_sdpa_gqa(nq, nkv):
    rng = np.random.default_rng(4)
    d = 16
    m = O.Model(_Shape(n_q=nq, n_kv=nkv, head_dim=d), _W())
    q = rng.standard_normal((9, nq, d))
    k = rng.standard_normal((23, nkv, d))
    v = rng.standard_normal((23, nkv, d))
    got = O.attention(m, q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    want = F.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    m = O.Model(_Shape(n_q=4, n_kv=2, head_dim=16), _W())
    k = rng.standard_normal((31, 2, 16))
    v = rng.standard_normal((31, 2, 16))
    # zero queries: uniform softmax, output = mean of the value rows of the mapped KV head
    out = O.attention(m, np.zeros((3, 4, 16)), k, v)
    for i in range(4):
        np.testing.assert_allclose(out[:, i], np.broadcast_to(v[:, i // 2].mean(0), (3, 16)), atol=1e-13)
    # a single key: output equals that value row
    out1 = O.attention(m, rng.standard_normal((2, 4, 16)), k[:1], v[:1])
    for i in range(4):
        np.testing.assert_allclose(out1[:, i], np.broadcast_to(v[0, i // 2], (2, 16)), atol=1e-14)
    # constant value rows per KV head identify the head map: query head i -> KV head floor(i*n_kv/n_q)
    vc = np.zeros((31, 2, 16))
    vc[:, 0] = 1.0
    vc[:, 1] = 7.0
    outc = O.attention(m, rng.standard_normal((3, 4, 16)), k, vc)
    np.testing.assert_allclose(outc[:, :, 0], np.array([[1, 1, 7, 7]] * 3, float), rtol=1e-13)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-300)
