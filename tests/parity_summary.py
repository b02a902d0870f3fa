"""Summarise the achieved-error records of a GPU test run as a markdown table.

The GPU tests append one JSON record per comparison to $CPATTN_PARITY_LOG
(tests/test_gpu_parity.py: record()). This groups the records by what was
compared and prints, for each group, the number of cases, the largest error
found and its tolerance:

    python tests/parity_summary.py parity_errors.jsonl > PARITY.md
"""
import json
import sys
from collections import OrderedDict


def rows_of(path):
    with open(path) as f:
        return [json.loads(line) for line in f if line.strip()]


def summarise(records):
    groups = OrderedDict()
    for r in records:
        # one group per comparison and tolerance (a name can cover both dtypes)
        tol = tuple(r.get(k) for k in ("o_tol", "lse_tol", "max_tol_rel"))
        groups.setdefault((r["test"], tol), []).append(r)
    out = ["| Compared | Cases | Checked | Worst error | Tolerance | Worst / tolerance |",
           "|---|---|---|---|---|---|"]
    worst_ratio = 0.0
    for (name, _), rs in groups.items():
        n_checked = sum(int(r.get("rows", r.get("elements", 0))) for r in rs)
        cells = []
        ratio = 0.0
        if "max_abs_err_o" in rs[0]:
            e = max(r["max_abs_err_o"] for r in rs)
            t = min(r["o_tol"] for r in rs)
            ratio = max(ratio, max(r["max_abs_err_o"] / r["o_tol"] for r in rs))
            cells.append(("O max abs %.2e" % e, "%.0e" % t))
        if "max_abs_err_lse" in rs[0]:
            e = max(r["max_abs_err_lse"] for r in rs)
            t = min(r["lse_tol"] for r in rs)
            ratio = max(ratio, max(r["max_abs_err_lse"] / r["lse_tol"] for r in rs))
            cells.append(("LSE max abs %.2e" % e, "%.1e" % t))
        if "max_abs_err" in rs[0]:
            rel = [r["max_abs_err"] / r["max_abs_ref"] for r in rs if r["max_abs_ref"] > 0]
            rms = [r["rms_err"] / r["rms_ref"] for r in rs if r["rms_ref"] > 0]
            zero = [r["max_abs_err"] for r in rs if r["max_abs_ref"] == 0]
            if rel:
                ratio = max(ratio, max(x / rs[0]["max_tol_rel"] for x in rel))
                cells.append(("max %.2e of max\\|g\\|" % max(rel), "%.0e" % rs[0]["max_tol_rel"]))
            if rms:
                ratio = max(ratio, max(x / rs[0]["rms_tol_rel"] for x in rms))
                cells.append(("rms %.2e of rms\\|g\\|" % max(rms), "%.0e" % rs[0]["rms_tol_rel"]))
            if zero:
                ratio = max(ratio, max(zero) / 1e-5)
                cells.append(("zero reference: %.2e abs" % max(zero), "1e-5"))
        worst_ratio = max(worst_ratio, ratio)
        out.append("| %s | %d | %d | %s | %s | %.2f |" % (name, len(rs), n_checked, "; ".join(c[0] for c in cells),
                                                          "; ".join(c[1] for c in cells), ratio))
    return out, worst_ratio


def main(path):
    records = rows_of(path)
    table, worst = summarise(records)
    print("%d comparisons; the largest error is %.2f of its tolerance.\n" % (len(records), worst))
    print("\n".join(table))


if __name__ == "__main__":
    main(sys.argv[1])
