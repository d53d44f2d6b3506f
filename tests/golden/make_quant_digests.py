"""Writes tests/golden/quant_720p_digests.json: the oracle's output for the whole
standalone quantize workload (40 heads x 75,600 tokens x d = 128, bf16 input drawn by
synth.quant_head: N(0,1), 3 outlier channels x16 per head, Bernoulli(0.001) spikes
x100), Hadamard-128 rotation then block quantisation along d, under UOS, OCP and
CEIL 6 (TFS).

For each rule and head it stores the SHA-256 of the packed codes ([75,600, 64]
bytes, even element in the low nibble) followed by the E8M0 scale bytes
([75,600, 4]), the layout mxattn_quantize writes.  Only the oracle and the seeded
input generator run here; nothing comes from the GPU path.

    python tests/golden/make_quant_digests.py      (about a minute on 8 cores)
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quant_720p_digests.json")
RULES = {"uos": ("ceil", 7.25), "ocp": ("ocp", None), "tfs": ("ceil", 6.0)}


def head_digests(h: int) -> dict:
    import synth
    from oracle import hadamard, mxfp4
    x = synth.quant_head(synth.QUANT_720P, h)
    y = hadamard.fwht_fp32(x)
    out = {}
    for name, rule in RULES.items():
        codes, scales = mxfp4.quantize_blocks_lastaxis(y, rule)
        d = hashlib.sha256()
        d.update(mxfp4.pack_nibbles(codes).tobytes())
        d.update(scales.astype("uint8").tobytes())
        out[name] = d.hexdigest()
    return out


def main():
    import synth
    w = synth.QUANT_720P
    with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        per_head = list(ex.map(head_digests, range(w.H)))
    doc = {
        "what": ("SHA-256 of mxfp4.pack_nibbles(codes) bytes then scale bytes, per head, of the oracle's "
                 "Hadamard-128 + block quantisation of the standalone quantize workload"),
        "workload": {"name": w.name, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype, "seed": w.seed},
        "source": ("oracle/hadamard.py fwht_fp32 and oracle/mxfp4.py quantize_blocks_lastaxis, written from "
                   "the Pith review of MXAttention (Axiom ledger axiom 1; Figure 3 caption for the scale rules)"),
        "generator": "tests/golden/make_quant_digests.py",
        "rules": {name: [ph[name] for ph in per_head] for name in RULES},
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
