"""Pins of the oracle's grouped output projection (oracle/project.py): a worked
example computed by hand, the one-group case as a single plain matrix product, and
the grouped result as one dense product with an explicitly block-diagonal weight
matrix (a grouping, head-order or transposition mistake fails at least one)."""
import os

import numpy as np

from oracle import project

GOLD = os.path.join(os.path.dirname(__file__), "golden", "grouped_projection_worked_example.txt")


def test_worked_example():
    line = [l for l in open(GOLD) if l.strip() and not l.startswith("#")][0]
    o, w0, w1, y = [np.array(p.split(), float) for p in line.split("|")]
    W = np.stack([w0.reshape(2, 4), w1.reshape(2, 4)])
    got = project.grouped_out_proj(o.reshape(1, 4, 2), W)
    assert np.array_equal(got.reshape(-1), y)


def test_one_group_is_a_plain_product():
    rng = np.random.default_rng(0)
    o = rng.normal(size=(5, 6, 8))
    W = rng.normal(size=(1, 7, 48))
    got = project.grouped_out_proj(o, W)[:, 0, :]
    want = np.einsum("nk,ck->nc", o.reshape(5, 48), W[0])
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_groups_are_a_block_diagonal_product():
    rng = np.random.default_rng(1)
    Nq, H, D, G, d_g = 3, 8, 4, 4, 5
    K_g = H // G * D
    o = rng.normal(size=(Nq, H, D))
    W = rng.normal(size=(G, d_g, K_g))
    big = np.zeros((G * d_g, H * D))             # block g maps inputs [g K_g, (g+1) K_g) to outputs [g d_g, ...)
    for g in range(G):
        big[g * d_g:(g + 1) * d_g, g * K_g:(g + 1) * K_g] = W[g]
    want = (o.reshape(Nq, H * D) @ big.T).reshape(Nq, G, d_g)
    assert np.allclose(project.grouped_out_proj(o, W), want, rtol=1e-13, atol=1e-13)
