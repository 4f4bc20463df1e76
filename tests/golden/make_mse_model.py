"""Writes mse_model_llama8.json: the three-term error model's per-element
non-max, max-element and zero-rounding terms for the narrow-Normal block-size
sweep (Llama-3.1-8B MLP shape, sigma in {0.002, 0.005, 0.01, 0.05}, blocks
256 ... 8, UE4M3 and UE5M3 scales without a per-tensor scale).

Calls only the oracle's model (oracle/mse_model.py; "Is finer better? Limits
of micro-scaling formats in LLMs", Framework Teorico).  The benchmark prints
these values beside the terms it measures on the GPU.

    python tests/golden/make_mse_model.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import mse_model  # noqa: E402

SIGMAS = (0.002, 0.005, 0.01, 0.05)
BLOCKS = (256, 128, 64, 32, 16, 8)
FORMATS = ("ue4m3", "ue5m3")


def table():
    out = {}
    for fmt in FORMATS:
        for s in SIGMAS:
            for b in BLOCKS:
                p = mse_model.predict(s, b, fmt)
                out[f"{fmt}/{s}/{b}"] = {k: p[k] for k in ("nonmax", "max", "zero", "total",
                                                          "p_zero_block")}
    return out


if __name__ == "__main__":
    path = os.path.join(HERE, "mse_model_llama8.json")
    json.dump({"source": "oracle/mse_model.py predict(sigma, block, fmt), g = 1; per-element "
                         "expected squared error of i.i.d. N(0, sigma) values",
               "terms": table()}, open(path, "w"), indent=1)
    print("wrote", path)
