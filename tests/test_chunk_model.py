"""The chunked (WY / UT) form of the gated delta rule, in fp64, equals the
token-by-token oracle for every chunk size, including partial last chunks and
chunk size 1 (where it reduces to the token step)."""
import numpy as np
import pytest

import oracle
from chunk_model import chunked_delta_rule


def _inputs(L, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True) * np.sqrt(dk)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, dv))
    g = -np.logaddexp(0, rng.standard_normal(L))
    b = 1 / (1 + np.exp(-rng.standard_normal(L)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    return q, k, v, g, b, S0


@pytest.mark.parametrize("chunk", [1, 2, 4, 7, 64])
def test_chunked_equals_token_loop(chunk):
    q, k, v, g, b, S0 = _inputs(150, 16, 12, chunk)
    o_ref, S_ref = oracle.delta_rule(q, k, v, g, b, S0)
    o, S = chunked_delta_rule(q, k, v, g, b, S0, chunk=chunk)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-10, atol=1e-12)


def test_bf16_operand_rounding_error_is_small():
    """Rounding every matrix-product operand to bf16 where the GPU kernel does
    keeps the relative L2 error of outputs and state well under 1e-2."""
    q, k, v, g, b, S0 = _inputs(2048, 128, 64, 99)
    q, k, v = [np.asarray(__import__("torch").from_numpy(a).to(__import__("torch").bfloat16).double()) for a in (q, k, v)]
    o_ref, S_ref = oracle.delta_rule(q, k, v, g, b, S0)
    o, S = chunked_delta_rule(q, k, v, g, b, S0, chunk=64, bf16=True)
    eo = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
    es = np.linalg.norm(S - S_ref) / np.linalg.norm(S_ref)
    assert eo < 3e-3 and es < 3e-3, (eo, es)
