"""Tabulate the parity margins of a GPU test run.

    RA_PARITY_LOG=<log.jsonl> python -m pytest tests -m gpu ...
    python tests/parity_margins.py <log.jsonl> > tests/parity_margins.md

Every comparison the GPU tests make against the oracle (tests/helpers.py,
assert_close) is one record: test id, tensor, max abs error, its bar and the
relative L2 error. The table lists, per test, the worst (largest error / bar)
record of each tensor kind, and the summary the tightest margins overall.
"""
import collections
import json
import re
import sys


def kind_of(tensor):
    """Tensor family of a record name ('dK chunk 3 g0' -> 'dK')."""
    m = re.match(r"(merged )?([A-Za-z]+)", tensor)
    return m.group(2) if m else tensor


def main(path):
    recs = [json.loads(l) for l in open(path) if l.strip()]
    worst = collections.OrderedDict()
    for r in recs:
        key = (r["test"], kind_of(r["tensor"]))
        ratio = r["max_abs"] / r["bar"] if r["bar"] else 0.0
        if key not in worst or ratio > worst[key][0]:
            worst[key] = (ratio, r)
    print("# Parity margins of the GPU tests against the fp64 oracle\n")
    print(f"Source: {len(recs)} comparisons recorded by `assert_close` (tests/helpers.py) in one "
          "run of `python -m pytest tests -m gpu` with `RA_PARITY_LOG` set; tabulated by "
          "`tests/parity_margins.py`. Bars: max abs error 2e-2 (O, dQ, dK, dV, D) and 1e-3 "
          "(LSE) for bf16, 1e-5 for fp32; rel-L2 < 1e-2 beside the bf16 value bar. "
          "`margin` = bar / max abs error (how many times the error fits under its bar).\n")
    by_kind = collections.defaultdict(list)
    for (test, kind), (ratio, r) in worst.items():
        by_kind[(kind, r["dtype"])].append((ratio, test, r))
    print("## Tightest case per tensor kind\n")
    print("| tensor | dtype | worst max abs | bar | margin | rel L2 | test |")
    print("|---|---|---|---|---|---|---|")
    for (kind, dt), lst in sorted(by_kind.items()):
        ratio, test, r = max(lst, key=lambda t: t[0])
        rl = "" if r["rel_l2"] is None else f"{r['rel_l2']:.2e}"
        margin = f"{1 / ratio:.1f}x" if ratio > 0 else "exact"
        print(f"| {kind} | {dt} | {r['max_abs']:.3e} | {r['bar']:.0e} | {margin} | {rl} | "
              f"`{test.split('::', 1)[-1]}` |")
    print("\n## Every test (worst record of each tensor kind)\n")
    print("| test | tensor | max abs | bar | margin | rel L2 |")
    print("|---|---|---|---|---|---|")
    for (test, kind), (ratio, r) in worst.items():
        rl = "" if r["rel_l2"] is None else f"{r['rel_l2']:.2e}"
        margin = f"{1 / ratio:.1f}x" if ratio > 0 else "exact"
        print(f"| `{test.split('::', 1)[-1]}` | {r['tensor']} | {r['max_abs']:.3e} | "
              f"{r['bar']:.0e} | {margin} | {rl} |")


if __name__ == "__main__":
    main(sys.argv[1])
