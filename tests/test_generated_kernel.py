"""The committed MFMA attention kernel source is exactly what its generator makes of the template:
regenerating decode_fast.hip from decode_fast.in.hip in memory must give the committed bytes."""

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_decode_decoupled_amd", "csrc")


def _generator():
    spec = importlib.util.spec_from_file_location("_gen_decode_fast", os.path.join(CSRC, "gen_decode_fast.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)   # the module writes nothing unless run as a script
    return mod


def test_decode_fast_matches_template():
    gen = _generator()
    want = gen.generate(os.path.join(CSRC, "decode_fast.in.hip"))
    with open(os.path.join(CSRC, "decode_fast.hip")) as fh:
        got = fh.read()
    assert got == want, "decode_fast.hip is stale: run gen_decode_fast.py after editing decode_fast.in.hip"
