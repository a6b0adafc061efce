"""The oracle's pins catch plausible mistakes: each mutation below is planted in an
in-memory copy of the oracle (the files are not touched), the pin tests of
test_oracle_pins.py run against that copy, and at least one of them must fail.
"""

import inspect
import os
import types

import pytest

import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REF_SRC = open(os.path.join(ROOT, "oracle", "reference.py")).read()
LAYOUT_SRC = open(os.path.join(ROOT, "oracle", "layout.py")).read()

# (module, original text, planted mistake)
MUTATIONS = {
    "nibble order": ("ref", "q[i::8] = (qweight >> np.uint32(4 * i))",
                     "q[i::8] = (qweight >> np.uint32(4 * (7 - i)))"),
    "zero-point lane order": ("ref", "z[:, i::8] = (zeros >> np.uint32(4 * i))",
                              "z[:, i::8] = (zeros >> np.uint32(4 * (7 - i)))"),
    "sign of q - z": ("ref", "return (qi - zi).astype(np.float64) * s[group, :]",
                      "return (zi - qi).astype(np.float64) * s[group, :]"),
    "group index": ("ref", "return np.arange(k, dtype=np.int64) // group_size",
                    "return np.arange(k, dtype=np.int64) % (k // group_size)"),
    "u4b8 offset": ("ref", "U4B8_ZERO = 8", "U4B8_ZERO = 7"),
    "act_order rows": ("ref", "        return g\n", "        return np.sort(g)\n"),
    "scale indexing": ("ref", "* s[group, :]", "* s[group % s.shape[0], ::-1]"),
    "CSR order": ("ref", "order = np.argsort(sel, kind=\"stable\")",
                  "order = np.argsort(-sel, kind=\"stable\")"),
    "bf16 decode": ("ref", "<< np.uint32(16)", "<< np.uint32(15)"),
    "bf16 rounding width": ("ref", "np.maximum(exp, -125) - 8)", "np.maximum(exp, -125) - 7)"),
    "bf16 subnormal spacing": ("ref", "np.maximum(exp, -125) - 8)", "exp - 8)"),
    "E4M3 bias": ("ref", "np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)"),
    "E4M3 subnormals": ("ref", "np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)"),
    "E4M3 word byte order": ("ref", "out[i::4, :] = (w >> np.uint32(8 * i))",
                             "out[i::4, :] = (w >> np.uint32(8 * (3 - i)))"),
    "block scale mapping": ("ref", "np.repeat(v, 128, axis=0).T",
                            "np.tile(v.T, (1, 128))"),
    "silu sign": ("ref", "x / (1.0 + np.exp(-x))", "x / (1.0 + np.exp(x))"),
    "SwiGLU fp16 activation unrounded": (
        "ref", "act16 = dequantize_fp16(swiglu_activation(a, gate, up, group_size=group_size))",
        "act16 = swiglu_activation(a, gate, up, group_size=group_size)"),
    "SwiGLU down projection zeros dropped": (
        "ref", "out = w4a16_gemm(act16, down[\"qweight\"], down[\"scales\"], zeros=down.get(\"zeros\"),",
        "out = w4a16_gemm(act16, down[\"qweight\"], down[\"scales\"], zeros=None,"),
    "SwiGLU bf16 activation unrounded": (
        "ref", "act = round_bf16(swiglu_activation(a, gate, up, group_size=group_size, bf16=True))",
        "act = swiglu_activation(a, gate, up, group_size=group_size, bf16=True)"),
    "SwiGLU bf16 down zeros dropped": (
        "ref", "w = w4a16_weights(down[\"qweight\"], down[\"scales\"], zeros=down.get(\"zeros\"),",
        "w = w4a16_weights(down[\"qweight\"], down[\"scales\"], zeros=None,"),
    "routing weight row": ("ref", "[rows].astype(np.float64)", "[rows[::-1]].astype(np.float64)"),
    "scale unit": ("layout", "        unit //= 2\n", "        unit //= 4\n"),
    "FP8 layout rows": ("layout", "+ 8 * qd + 4 * (d % 2) + i", "+ 4 * qd + 8 * (d % 2) + i"),
    "nibble slot order": ("layout", "SLOT = (0, 4, 1, 5, 2, 6, 3, 7)",
                          "SLOT = (0, 1, 2, 3, 4, 5, 6, 7)"),
}


def load(src: str, name: str, ref_module=None) -> types.ModuleType:
    mod = types.ModuleType(name)
    if ref_module is not None:  # layout.py imports the reference module relatively
        src = src.replace("from .reference import unpack_qweight",
                          "unpack_qweight = _ref.unpack_qweight")
        mod._ref = ref_module
    exec(compile(src, name, "exec"), mod.__dict__)
    return mod


def failing_pin(monkeypatch, ref_mod, layout_mod):
    monkeypatch.setattr(pins, "ref", ref_mod)
    monkeypatch.setattr(pins, "layout", layout_mod)
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if name.startswith("test_") and not inspect.signature(fn).parameters:
            try:
                fn()
            except Exception:
                return name
    return None


def test_unmutated_copies_pass_every_pin(monkeypatch):
    ref_mod = load(REF_SRC, "reference_copy")
    assert failing_pin(monkeypatch, ref_mod, load(LAYOUT_SRC, "layout_copy", ref_mod)) is None


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(monkeypatch, mutation):
    where, original, planted = MUTATIONS[mutation]
    src = REF_SRC if where == "ref" else LAYOUT_SRC
    assert src.count(original) >= 1, f"{mutation}: text to mutate not found"
    mutated = src.replace(original, planted)
    if where == "ref":
        ref_mod = load(mutated, "reference_mutant")
        layout_mod = load(LAYOUT_SRC, "layout_copy", ref_mod)
    else:
        ref_mod = load(REF_SRC, "reference_copy")
        layout_mod = load(mutated, "layout_mutant", ref_mod)
    caught = failing_pin(monkeypatch, ref_mod, layout_mod)
    assert caught is not None, f"no pin fails with the mistake '{mutation}'"
