import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # A gpu-marked test never silently passes on a CPU-only host: it is skipped
    # when no GPU is visible, and the product path itself raises if the HIP
    # library is missing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """Writes the per-workload error table (max and mean |GPU - oracle| of
    each output over everything compared) to the file FA_PARITY_LOG names."""
    path = os.environ.get("FA_PARITY_LOG")
    if not path:
        return
    import json
    from tests.util import RECORDS
    table = {}
    for r in RECORDS:
        e = table.setdefault((r["config"], r["output"]), {"max_abs": 0.0, "sum_abs": 0.0, "n": 0})
        e["max_abs"] = max(e["max_abs"], r["max_abs"])
        e["sum_abs"] += r["sum_abs"]
        e["n"] += r["n"]
    rows = [{"config": c, "output": o, "max_abs": e["max_abs"], "mean_abs": e["sum_abs"] / e["n"],
             "elements": e["n"]} for (c, o), e in sorted(table.items())]
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"exitstatus": int(exitstatus), "rows": rows}, f, indent=1)
    with open(os.path.splitext(path)[0] + ".md", "w") as f:
        f.write(error_table_markdown(rows, int(exitstatus)))


def error_table_markdown(rows, exitstatus):
    """The error table as Markdown (one row per workload and output)."""
    out = ["| workload | output | elements compared | max abs err | mean abs err |",
           "|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %s | %d | %.3g | %.3g |" % (r["config"], r["output"], r["elements"],
                                                       r["max_abs"], r["mean_abs"]))
    return "\n".join(out) + "\n\n(pytest exit status %d)\n" % exitstatus
