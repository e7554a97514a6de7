"""Write tests/golden/synth_sha256.json: SHA-256 of small generated tensors.

Calls only the seeded generator (``synth``); it pins the generator's bytes so a
change to it cannot pass unnoticed. Run from the repository root:
    python tests/golden/make_synth_digests.py
"""
import hashlib
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import synth  # noqa: E402

CASES = {
    "normal_bf16(0,'gpt2.A',(8,768))": lambda: synth.normal_bf16(0, "gpt2.A", (8, 768)),
    "normal_bf16(1,'gemv.W',(64,4096),0.02)": lambda: synth.normal_bf16(1, "gemv.W", (64, 4096), 0.02),
    "rademacher(0,'gemv.r',4096)": lambda: synth.rademacher(0, "gemv.r", 4096),
    "integer_bf16(0,'int.A',(33,300))": lambda: synth.integer_bf16(0, "int.A", (33, 300)),
}


def digests():
    return {k: hashlib.sha256(f().tobytes()).hexdigest() for k, f in CASES.items()}


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "synth_sha256.json")
    json.dump(digests(), open(out, "w"), indent=1)
    print(out)
