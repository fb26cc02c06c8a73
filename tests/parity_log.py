"""Counts of near-tie token differences seen by the GPU parity tests.

``check_rows`` records, per checked verify, the rows compared, the argmax
differences at an oracle gap of at most one bf16 ulp (ties), the wider ones
backed by the oracle's unrounded run (flips) and the logit error against its
tolerance.  When the environment variable TV_PARITY_LOG names a file, the
records are written there as JSON at the end of the session.
"""
import json
import os

RECORDS = []


def record(what, rows, ties, flips, max_abs_dlogit, tol_min, tol_max):
    RECORDS.append({"case": what, "rows": int(rows), "ties": int(ties), "flips": int(flips),
                    "max_abs_dlogit": max_abs_dlogit, "tol_min": tol_min, "tol_max": tol_max})


def write():
    path = os.environ.get("TV_PARITY_LOG")
    if not path or not RECORDS:
        return
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    tot = {k: sum(r[k] for r in RECORDS) for k in ("rows", "ties", "flips")}
    with open(path, "w") as f:
        json.dump({"total": tot, "records": RECORDS}, f, indent=1)


def render(path, commit, passed):
    """Markdown table of a written log: ``python tests/parity_log.py LOG COMMIT PASSED``."""
    d = json.load(open(path))
    tot = d["total"]
    out = ["| case | rows | ties | flips | max abs logit error | tolerance (min .. max over rows) |",
           "|---|---:|---:|---:|---:|---|"]
    for r in d["records"]:
        out.append(f"| {r['case']} | {r['rows']} | {r['ties']} | {r['flips']} | {r['max_abs_dlogit']:.4g} | "
                   f"{r['tol_min']:.4g} .. {r['tol_max']:.4g} |")
    head = (f"on MI355X at commit `{commit}` ({passed} GPU tests passed).",
            f"**Total: {tot['rows']} rows compared, {tot['ties']} ties, {tot['flips']} flips.**")
    return head, "\n".join(out)


if __name__ == "__main__":
    import sys
    head, table = render(sys.argv[1], sys.argv[2], sys.argv[3])
    print(head[0]); print(head[1]); print(); print(table)
