"""Pins of the decoder oracle (oracle.model) against facts outside it.

* GELU against the standard normal CDF at printed table values and the
  identity gelu(x) - gelu(-x) = x;
* RMSNorm on constant vectors (closed form) and its scale invariance;
* the whole model against a pure-Python brute force (math.fsum loops) on a
  tiny configuration;
* incremental decoding through the cache equals the full forward at every
  position (the README's cached-equals-uncached claim), and later tokens never
  change earlier logits.

Each check takes the functions under test as arguments, and the mutation test
at the end plants plausible mistakes in copies and shows that a check fails.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
import synth_inputs as si

TINY = dataclasses.replace(si.TINYGPT, layers=2, d_model=8, heads=2, vocab=11, max_T=8)
SMALL = dataclasses.replace(si.TINYGPT, layers=2, d_model=64, heads=4, vocab=97, max_T=24)


def check_gelu(gelu=oracle.model.gelu):
    # Phi(1) = 0.8413447460685429, Phi(-1) = 0.15865525393145707, Phi(2) = 0.9772498680518208
    assert gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(gelu(np.array([1.0, -1.0, 2.0])),
                               [0.8413447460685429, -0.15865525393145707, 2 * 0.9772498680518208], rtol=1e-14)
    x = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(gelu(x) - gelu(-x), x, atol=1e-14)
    assert abs(gelu(np.array([-12.0]))[0]) < 1e-30 and gelu(np.array([12.0]))[0] == 12.0


def check_rmsnorm(rmsnorm=oracle.model.rmsnorm):
    g = np.array([1.0, 2.0, -0.5, 3.0])
    for c in (0.25, -3.0, 40.0):
        got = rmsnorm(np.full(4, c), g)
        np.testing.assert_allclose(got, g * c / math.sqrt(c * c + 1e-5), rtol=1e-14)
    x = np.random.default_rng(3).standard_normal((5, 16)) * 7.0
    y = rmsnorm(x, np.ones(16))
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-6)
    np.testing.assert_allclose(rmsnorm(1000.0 * x, np.ones(16)), y, rtol=1e-6)  # eps / (2 mean(x^2)) ~ 1e-7


def brute_logits(spec, w, tokens):
    """Pure-Python loops: one sequence, every position, float64 via math.fsum."""
    d, H = spec.d_model, spec.heads
    D = d // H
    scale = float(np.float32(1.0 / math.sqrt(D)))
    f = lambda a: [float(v) for v in np.asarray(a, np.float64).reshape(-1)]
    mat = lambda name: [f(row) for row in np.asarray(w[name], np.float64)]
    vec = lambda name: f(w[name])
    h16 = lambda v: float(np.float16(v))

    def norm(x, gain):
        r = math.sqrt(math.fsum(v * v for v in x) / len(x) + 1e-5)
        return [x[i] / r * gain[i] for i in range(len(x))]

    def matvec(m, x):
        return [math.fsum(m[o][i] * x[i] for i in range(len(x))) for o in range(len(m))]

    T = len(tokens)
    tok, pos = mat("tok_emb"), mat("pos_emb")
    xs = [[tok[tokens[t]][i] + pos[t][i] for i in range(d)] for t in range(T)]
    for l in range(spec.layers):
        ln1, wqkv, wo = vec(f"ln1.{l}"), mat(f"wqkv.{l}"), mat(f"wo.{l}")
        ln2, wup, wdown = vec(f"ln2.{l}"), mat(f"w_up.{l}"), mat(f"w_down.{l}")
        qkv = [matvec(wqkv, norm(x, ln1)) for x in xs]
        new = []
        for t in range(T):
            att = []
            for h in range(H):
                q = [h16(qkv[t][h * D + e]) for e in range(D)]
                keys = [[h16(qkv[j][d + h * D + e]) for e in range(D)] for j in range(t + 1)]
                vals = [[h16(qkv[j][2 * d + h * D + e]) for e in range(D)] for j in range(t + 1)]
                s = [scale * math.fsum(q[e] * keys[j][e] for e in range(D)) for j in range(t + 1)]
                top = max(s)
                p = [math.exp(v - top) for v in s]
                z = math.fsum(p)
                att += [math.fsum(p[j] * vals[j][e] for j in range(t + 1)) / z for e in range(D)]
            x = [xs[t][i] + o for i, o in enumerate(matvec(wo, att))]
            hid = [0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0))) for u in matvec(wup, norm(x, ln2))]
            new.append([x[i] + o for i, o in enumerate(matvec(wdown, hid))])
        xs = new
    lnf, head = vec("ln_f"), mat("lm_head")
    return np.array([matvec(head, norm(x, lnf)) for x in xs])


def check_brute(forward=oracle.model.forward):
    w = si.model_weights(TINY, seed=1)
    tokens = si.model_tokens(TINY, 1, 6, seed=1)
    got = forward(TINY, w, tokens)[0]
    np.testing.assert_allclose(got, brute_logits(TINY, w, [int(t) for t in tokens[0]]), rtol=1e-11, atol=1e-12)


def check_incremental_equals_full(forward=oracle.model.forward, Decoder=oracle.model.Decoder):
    w = si.model_weights(SMALL, seed=2)
    tokens = si.model_tokens(SMALL, 2, 20, seed=2)
    full = forward(SMALL, w, tokens)
    dec = Decoder(SMALL, w, 2)
    np.testing.assert_allclose(dec.prefill(tokens[:, :9]), full[:, 8], rtol=1e-11, atol=1e-12)
    for t in range(9, 20):
        np.testing.assert_allclose(dec.step(tokens[:, t]), full[:, t], rtol=1e-11, atol=1e-12)


def check_causality(forward=oracle.model.forward):
    w = si.model_weights(SMALL, seed=3)
    tokens = si.model_tokens(SMALL, 1, 12, seed=3)
    other = tokens.copy()
    other[0, 7:] = (other[0, 7:] + 5) % SMALL.vocab
    a, b = forward(SMALL, w, tokens), forward(SMALL, w, other)
    assert np.array_equal(a[:, :7], b[:, :7]) and not np.allclose(a[:, 7:], b[:, 7:])


def test_gelu():
    check_gelu()


def test_rmsnorm():
    check_rmsnorm()


def test_brute():
    check_brute()


def test_incremental_equals_full():
    check_incremental_equals_full()


def test_causality():
    check_causality()


# ------------------------------------------------------------------ mutants
def _tanh_gelu(x):
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _layernorm(x, gain):
    x = np.asarray(x, np.float64)
    x = x - x.mean(axis=-1, keepdims=True)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-5) * gain


def _forward_with(**patch):
    """oracle.model.forward with some module-level functions replaced."""
    def fwd(spec, w, tokens):
        saved = {k: getattr(oracle.model, k) for k in patch}
        try:
            for k, v in patch.items():
                setattr(oracle.model, k, v)
            return oracle.model.forward(spec, w, tokens)
        finally:
            for k, v in saved.items():
                setattr(oracle.model, k, v)
    return fwd


def _decoder_pos_off_by_one():
    class D(oracle.model.Decoder):
        def step(self, tokens):
            self.pos += 1
            out = super().step(tokens)
            self.pos -= 1
            return out
    return D


def _interleaved_heads(x, H):
    B, T, d = x.shape
    return x.reshape(B, T, d // H, H).transpose(0, 3, 1, 2)


MUTANTS = {
    "gelu_tanh_approximation": lambda: check_gelu(_tanh_gelu),
    "layernorm_instead_of_rmsnorm": lambda: check_rmsnorm(_layernorm),
    "layernorm_in_the_model": lambda: check_brute(_forward_with(rmsnorm=_layernorm)),
    "heads_interleaved": lambda: check_brute(_forward_with(_heads=_interleaved_heads)),
    "no_storage_rounding": lambda: check_brute(_forward_with(_to_storage=lambda x: np.asarray(x, np.float64))),
    "decode_position_off_by_one": lambda: check_incremental_equals_full(
        oracle.model.forward, _decoder_pos_off_by_one()),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with pytest.raises(AssertionError):
        MUTANTS[name]()
