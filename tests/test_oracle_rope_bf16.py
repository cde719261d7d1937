"""Pins for the oracle's rotary embedding and bf16 rounding (CPU only).

RoPE: AstrAI docs/developer/internals.md, "Rotary Position Embedding (RoPE)" --
q_i^T k_j depends only on i - j; the rotation is a complex multiplication
(docs/guides/inference.md, "Rotary Embedding Backend": view as complex,
multiply, view as real); theta = 10 000 (AstrAI paper, "Model Architecture").
bf16: AstrAI paper, "BF16 dead zone" -- 7-bit mantissa, ulp 2^-7 at 1.0.
"""

import numpy as np
import pytest
import torch

from oracle import bf16, rope

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


@pytest.mark.parametrize("d", [64, 128])
def test_relative_position_invariance(d):
    rng = np.random.default_rng(0)
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    for i, j, s in [(0, 0, 5), (7, 3, 100), (3, 7, 2048), (31, 1, 32000), (1000, 999, 31000)]:
        base = rope.rotate(q, i) @ rope.rotate(k, j)
        shifted = rope.rotate(q, i + s) @ rope.rotate(k, j + s)
        # float64 angles carry ~eps * position of absolute error
        tol = 4e-16 * (1 + i + j + 2 * s) * np.linalg.norm(q) * np.linalg.norm(k)
        assert abs(base - shifted) <= tol


def test_relative_dependence_is_real():
    # a different offset i - j gives a different score (guards a no-op rotation)
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = rope.rotate(q, 5) @ rope.rotate(k, 2)
    b = rope.rotate(q, 6) @ rope.rotate(k, 2)
    assert abs(a - b) > 1e-3


def test_norm_preserved_and_position_zero_is_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 4, 128))
    pos = rng.integers(0, 32768, size=(9, 1))
    y = rope.rotate(x, pos)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    z = rope.rotate(x, np.zeros((9, 1)))
    assert np.array_equal(z, x)


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_complex_multiplication_of_adjacent_pairs(d):
    # numpy's complex view of a float64 array pairs (x[2i], x[2i+1]) exactly as
    # torch.view_as_complex does on [..., D/2, 2]; multiplying by e^{i*angle}
    # fixes both the pair layout and the direction of rotation.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, d))
    pos = np.array([0, 1, 2, 17, 2047, 32767])
    z = x.copy().view(np.complex128)                      # [6, d/2]
    freq = 10000.0 ** (-np.arange(0, d, 2) / d)
    expect = (z * np.exp(1j * pos[:, None] * freq[None, :])).view(np.float64)
    np.testing.assert_allclose(rope.rotate(x, pos), expect, rtol=0, atol=1e-12)
    # the same against torch's complex path on the CPU
    tx = torch.from_numpy(x).reshape(6, d // 2, 2)
    tz = torch.view_as_complex(tx.contiguous())
    tf = torch.polar(torch.ones(6, d // 2, dtype=torch.float64),
                     torch.from_numpy(pos[:, None] * freq[None, :]))
    ty = torch.view_as_real(tz * tf).reshape(6, d).numpy()
    np.testing.assert_allclose(rope.rotate(x, pos), ty, rtol=0, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_frequencies_are_the_roformer_progression(d):
    # at position 1 pair i turns by theta^(-2i/d): 1 for the first pair, a constant
    # ratio theta^(-2/d) between neighbours, theta^(-(d-2)/d) for the last.
    f = rope.inv_freq(d, 10000.0)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[1:] / f[:-1], 10000.0 ** (-2.0 / d), rtol=1e-14)
    np.testing.assert_allclose(f[-1], 10000.0 ** (-(d - 2) / d), rtol=1e-14)
    e = np.zeros(d)
    e[0::2] = 1.0                                          # every pair = 1 + 0i
    y = rope.rotate(e, 1)
    ang = np.arctan2(y[1::2], y[0::2])
    np.testing.assert_allclose(ang, f, rtol=0, atol=1e-14)


def test_freqs_table_matches_rotation():
    d, n = 128, 300
    tab = rope.freqs_cis(n, d)
    assert tab.shape == (n, d // 2, 2)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((n, d))
    z = x.copy().view(np.complex128) * (tab[..., 0] + 1j * tab[..., 1])
    np.testing.assert_allclose(rope.rotate(x, np.arange(n)), z.view(np.float64),
                               rtol=0, atol=1e-12)


def test_rotation_by_the_stored_float32_table():
    # with the float64 table the lookup form equals the exact rotation; with the
    # float32 table it differs by at most the table's rounding (2^-24 relative
    # per entry), and the float32 table is the float64 one rounded to nearest
    d, n = 128, 4096
    rng = np.random.default_rng(6)
    x = rng.standard_normal((n, 4, d))
    pos = rng.integers(0, n, size=(n, 1))
    np.testing.assert_allclose(rope.rotate_with_table(x, pos, rope.freqs_cis(n, d)),
                               rope.rotate(x, pos), rtol=0, atol=1e-12)
    t32 = rope.freqs_cis_f32(n, d)
    t64 = rope.freqs_cis(n, d)
    assert np.array_equal(t32, t64.astype(np.float32).astype(np.float64))
    assert np.all(np.abs(t32 - t64) <= np.spacing(np.abs(t64).astype(np.float32)) / 2)
    err = np.abs(rope.rotate_with_table(x, pos, t32) - rope.rotate(x, pos))
    bound = 2.0 ** -24 * (np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]))
    assert np.all(err[..., 0::2] <= bound) and np.all(err[..., 1::2] <= bound)
    assert err.max() > 0                       # the stored table is not the exact one


# -- gradient of the rotation -------------------------------------------------------

def test_rotation_gradient_equals_torch_autograd():
    # the complex-multiply forward differentiated by torch's autograd (float64,
    # the table entries as complex numbers) gives the oracle's gradient
    d, n = 128, 64
    rng = np.random.default_rng(7)
    table = rope.freqs_cis_f32(4096, d)
    pos = rng.integers(0, 4096, size=n)
    x = rng.standard_normal((n, 3, d))
    g = rng.standard_normal((n, 3, d))
    xt = torch.tensor(x, requires_grad=True)
    tt = torch.tensor(table[pos])                                    # [n, d/2, 2]
    rot = torch.complex(tt[..., 0], tt[..., 1])[:, None, :]          # [n, 1, d/2]
    y = torch.view_as_real(torch.view_as_complex(xt.reshape(n, 3, d // 2, 2)) * rot).reshape(n, 3, d)
    y.backward(torch.tensor(g))
    want = xt.grad.numpy()
    np.testing.assert_allclose(rope.rotate_with_table(x, pos[:, None], table), y.detach().numpy(),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(rope.rotate_backward_with_table(g, pos[:, None], table), want,
                               rtol=0, atol=1e-12)


def test_rotation_gradient_is_the_adjoint_and_undoes_the_rotation():
    # <R x, g> = <x, R^T g>; with the exact float64 table R^T R = I and the
    # gradient rotation is the rotation by -pos
    d, n = 64, 500
    rng = np.random.default_rng(8)
    table = rope.freqs_cis_f32(1000, d)
    pos = rng.integers(0, 1000, size=(n, 1))
    x = rng.standard_normal((n, 2, d))
    g = rng.standard_normal((n, 2, d))
    lhs = np.sum(rope.rotate_with_table(x, pos, table) * g)
    rhs = np.sum(x * rope.rotate_backward_with_table(g, pos, table))
    assert abs(lhs - rhs) <= 1e-10 * np.sum(np.abs(x) * np.abs(g))
    exact = rope.freqs_cis(1000, d)
    back = rope.rotate_backward_with_table(rope.rotate_with_table(x, pos, exact), pos, exact)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rope.rotate_backward_with_table(g, pos, exact), rope.rotate(g, -pos),
                               rtol=0, atol=1e-12)


# -- bf16 -----------------------------------------------------------------------

def test_round_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e4).astype(np.float32),
        (rng.standard_normal(20000) * 1e-4).astype(np.float32),
    ])
    # exact ties: bf16 value + half a bf16 ulp, both mantissa parities
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy().astype(np.float64)
    ties = (base + bf16.ulp_bf16(base) / 2).astype(np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = bf16.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_ties_and_ulp():
    assert bf16.ulp_bf16(1.0) == 2.0 ** -7                  # the paper's figure
    assert bf16.ulp_bf16(1.99) == 2.0 ** -7
    assert bf16.ulp_bf16(2.0) == 2.0 ** -6
    assert bf16.ulp_bf16(-0.75) == 2.0 ** -8
    assert bf16.round_bf16(1.0 + 2.0 ** -8) == 1.0          # tie -> even mantissa
    assert bf16.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert bf16.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert bf16.round_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert bf16.round_bf16(0.0) == 0.0
