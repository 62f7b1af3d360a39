"""Plausible mistakes planted in copies of the oracle (on the CPU) must each
be caught by the pin battery: this shows the pins constrain every part of
the oracle that the GPU path is compared against."""

import os
import types

import pytest

from tests.oracle_pins import ALL_CHECKS
from tests.test_oracle_fp8 import FP8_CHECKS
from tests.test_oracle_mods import MOD_CHECKS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")
SRC_FP8 = os.path.join(os.path.dirname(SRC), "fp8.py")

MUTATIONS = {
    "gqa head map h % Hkv": ("g = h // group", "g = h % Hkv"),
    "causal off by one": ("j[None, :] <= pos[:, None]", "j[None, :] < pos[:, None]"),
    "window off by one": ("(pos[:, None] - j[None, :]) < window", "(pos[:, None] - j[None, :]) <= window"),
    "top-left causal alignment": ("pos = rows + (skv - sq)", "pos = rows"),
    "scale dropped": ("s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T)"),
    "lse without max": ("m_safe + np.log(np.where(empty, 1.0, l))", "np.log(np.where(empty, 1.0, l))"),
    "no normalisation": ("num / np.where(empty, 1.0, l)[:, None]", "num"),
    "combine lse without max": ("M_safe + np.log(np.where(empty, 1.0, tot))", "np.log(np.where(empty, 1.0, tot))"),
    "combine unnormalised weights": ("w / np.where(empty, 1.0, tot)[..., None]", "w"),
    "gather slot index": ("out[b, t] = cache[page, t % page_size]", "out[b, t] = cache[page, t // page_size % page_size]"),
    "seq_lens ignored": ("skv = seq_lens[b]", "skv = Skv"),
    "empty row lse": ("lse = np.where(empty, -np.inf,", "lse = np.where(empty, 0.0,"),
    'softcap after bias': ('    if softcap > 0:\n        s = softcap * np.tanh(s / softcap)\n    if bias is not None:\n        s = s + bias',
        '    if bias is not None:\n        s = s + bias\n    if softcap > 0:\n        s = softcap * np.tanh(s / softcap)'),
    'softcap without inner division': ('s = softcap * np.tanh(s / softcap)',
        's = softcap * np.tanh(s)'),
    'alibi sign flipped': ('bias = slopes[h] * (np.arange(skv)[None, :] - pos[:, None])',
        'bias = slopes[h] * (pos[:, None] - np.arange(skv)[None, :])'),
    'alibi head off by one': ('m0 ** (h + 1) if h < n',
        'm0 ** h if h < n'),
    'alibi second ramp': ('m1 ** (2 * (h - n) + 1)',
        'm1 ** (h - n + 1)'),
    'sink missing from denominator': ('l = e.sum(axis=1) + np.exp(sink - m_safe)',
        'l = e.sum(axis=1)'),
    'sink missing from max': ('m = np.maximum(m, sink)',
        'm = m'),
    'mask ignored': ('        s = s + mask\n', '        s = s\n'),
    'mask subtracted': ('        s = s + mask\n', '        s = s - mask\n'),
    'mask of the first sequence for all': ('mask_v[b if mask_v.shape[0] > 1 else 0]', 'mask_v[0]'),
    'mask rows reversed': ('[rr, :skv]', '[rr[::-1], :skv]'),
    'value width taken from the key width': ('    Dv = v.shape[3]\n', '    Dv = q.shape[3]\n'),
    'mask keys shifted in decode': ('mask = mask[:, :, :kmax] if', 'mask = np.roll(mask, 1, axis=2)[:, :, :kmax] if'),
}


def _load_mutant(old, new, path=SRC):
    with open(path) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_battery():
    import oracle
    for check in ALL_CHECKS + MOD_CHECKS:
        check(oracle)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod = _load_mutant(*MUTATIONS[name])
    caught = []
    for check in ALL_CHECKS + MOD_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"mutation '{name}' passed every pin"


FP8_MUTATIONS = {
    "exponent bias 8": ("2.0 ** (e - 7)", "2.0 ** (e - 8)"),
    "subnormal scale": ("2.0 ** (1 - 7)", "2.0 ** (0 - 7)"),
    "implicit one on subnormals": ("return sign * (m / 8.0) * 2.0 ** (1 - 7)", "return sign * (1.0 + m / 8.0) * 2.0 ** (1 - 7)"),
    "ties away from zero": ("np.where(lo % 2 == 0, lo, hi)", "hi"),
    "ties toward zero": ("np.where(lo % 2 == 0, lo, hi)", "lo"),
    "sign dropped": ("codes | 0x80", "codes"),
    "append token off by one": ("            t = n - snew + i\n", "            t = n - snew + i + 1\n"),
    "append ignores the head scale": ("kq = quantize_e4m3(kn / ks[None, None, :, None])", "kq = quantize_e4m3(kn / ks[0])"),
    "dequantise with head 0's scale for every head": ("return vals * scale[:, None]", "return vals * scale[0]"),
    "dequantise with the scale broadcast along D": ("return vals * scale[:, None]",
                                                   "return vals * np.resize(scale, vals.shape[-1])"),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTATIONS))
def test_fp8_mutation_is_caught(name):
    mod = _load_mutant(*FP8_MUTATIONS[name], path=SRC_FP8)
    caught = []
    for check in FP8_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"mutation '{name}' passed every pin"
