"""The SwiGLU tables the library compiles in, against the oracle, entry by entry.

gen_silu_tables.py (the library's build step) evaluates s_g = RN32(g / RN32(1 +
RN32(e^-g))) and ds = silu'(g) exactly on rationals for every bf16 gate value in
the tabulated exponent range; the oracle computes the same steps in C with fp32
operations (swiglu_grad_one with u = dh = 1 gives du = s_g and dg = ds).  Every
one of the 2 x 8704 bit patterns must agree.
"""
import importlib.util
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_generator():
    path = os.path.join(ROOT, "fp8_precision_amd", "csrc", "gen_silu_tables.py")
    spec = importlib.util.spec_from_file_location("gen_silu_tables", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_generated_tables_match_the_oracle(orc):
    gen = load_generator()
    sg, ds = gen.entries()
    assert len(sg) == len(ds) == 2 * (gen.E_HI - gen.E_LO + 1) * 128
    i = 0
    bad = []
    one = np.float32(1.0)
    for sign in (0, 1):
        for ex in range(gen.E_LO, gen.E_HI + 1):
            for man in range(128):
                g = np.array([((sign << 15) | (ex << 7) | man) << 16], np.uint32).view(np.float32)[0]
                dg, du = orc.swiglu_grad_one(g, one, one)
                want_sg = int(np.float32(du).view(np.uint32))
                want_ds = int(np.float32(dg).view(np.uint32))
                if sg[i] != want_sg or ds[i] != want_ds:
                    bad.append((hex(int(g.view(np.uint32)) >> 16), hex(sg[i]), hex(want_sg), hex(ds[i]), hex(want_ds)))
                i += 1
    assert not bad, f"{len(bad)} entries differ, first: {bad[:4]}"


def test_rn32_rounding_cases():
    """The generator's binary32 rounding on values whose rounding is known."""
    from fractions import Fraction as Fr
    rn = load_generator().rn32
    assert rn(Fr(1)) == 0x3F800000
    assert rn(Fr(-2)) == 0xC0000000
    assert rn(1 + Fr(1, 2 ** 24)) == 0x3F800000                       # tie -> even (down)
    assert rn(1 + Fr(3, 2 ** 24)) == 0x3F800002                       # tie -> even (up)
    assert rn(1 + Fr(1, 2 ** 24) + Fr(1, 2 ** 60)) == 0x3F800001      # just above the tie
    assert rn(Fr(1, 2 ** 149)) == 0x00000001                          # smallest subnormal
    assert rn(Fr(1, 2 ** 150)) == 0                                   # tie with 0 -> even
    assert rn(Fr(3, 2 ** 151)) == 0x00000001
    assert rn(Fr(2) ** 128) == 0x7F800000                             # overflow -> inf
    assert rn(Fr(2) ** 127 * (2 - Fr(1, 2 ** 23))) == 0x7F7FFFFF     # largest finite
    assert rn(Fr(1, 3)) == int(np.float32(1 / 3).view(np.uint32))
