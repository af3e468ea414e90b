"""Parity margins table from the JSON lines the GPU tests append when KDA_MARGINS_OUT is
set (one line per checked tensor: test id, tensor, rel_err, bar):

    KDA_MARGINS_OUT=gpurun_out/margins.jsonl python -m pytest tests -m gpu -k "<tests>"
    python tests/margins_table.py gpurun_out/margins.jsonl

prints a markdown table: rel_err, the bar, and the margin (bar / rel_err)."""
import json
import sys


def main(path):
    rows = [json.loads(l) for l in open(path) if l.strip()]
    print("| test | tensor | rel_err | bar | margin (bar / rel_err) |")
    print("|---|---|---|---|---|")
    for r in rows:
        m = r["bar"] / r["rel_err"] if r["rel_err"] > 0 else float("inf")
        test = r["test"].split("::", 1)[-1]
        print("| %s | %s | %.2e | %.0e | %.1f |" % (test, r["tensor"], r["rel_err"], r["bar"], m))


if __name__ == "__main__":
    main(sys.argv[1])
