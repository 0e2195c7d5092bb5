"""Turn the JSON lines that test_gpu_full_size.py appends to $FA_PARITY_RECORD into a
markdown table (one row per workload and output tensor).

    python tests/parity_table.py parity.jsonl > table.md
"""

import json
import sys

ORDER = ["O", "lse", "dQ", "dK", "dV"]


def table(path):
    rows = [json.loads(line) for line in open(path) if line.strip()]
    out = ["| workload | shape (B, Hq/Hkv, Nq/Nk, d) | dtype | causal | launch | tensor | raw max | mean | "
           "rounding floor max | beyond floor max | max abs ref |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        B, H, Hkv, N, Nk, d = r["shape"]
        shape = f"{B}, {H}" + (f"/{Hkv}" if Hkv != H else "") + f", {N}" + (f"/{Nk}" if Nk != N else "") + f", {d}"
        launch = ("split " + str(r["split"])) if r["split"] > 1 else "one pass"
        if r["block_mask"]:
            launch += ", block mask"
        for key in ORDER:
            e = r["errors"].get(key)
            if e is None:
                continue
            if key == "lse":
                out.append(f"| {r['workload']} | {shape} | {r['dtype']} | {'yes' if r['causal'] else 'no'} | {launch} "
                           f"| lse (relative) | {e['max']:.2e} | {e['mean']:.2e} | — | — | {e['max_abs_ref']:.2f} |")
            else:
                out.append(f"| {r['workload']} | {shape} | {r['dtype']} | {'yes' if r['causal'] else 'no'} | {launch} "
                           f"| {key} | {e['max']:.2e} | {e['mean']:.2e} | {e['floor_max']:.2e} | "
                           f"{e['beyond_floor_max']:.2e} | {e['max_abs_ref']:.2f} |")
    return "\n".join(out)


if __name__ == "__main__":
    print(table(sys.argv[1]))
