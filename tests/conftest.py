import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case")


# full-size parity cases whose figures the session summary prints, by test function
FULL_SIZE = (
    ("test_gpt_oss_layer_full_oracle", "gptoss-T4096"),
    ("test_lora_full_size", "gptoss-T4096-lora16"),
    ("test_ep_rank_share_full_oracle", "ep-share-8192"),
    ("test_gpt_oss_layer_zipf_skew_sampled", "gptoss-zipf-T16384"),
    ("test_qwen3_layer_sampled", "qwen3-T32768"),
    ("test_expert_with_more_than_2_pow_31", "one-expert-2^31"),
)


def _label(test_id):
    for fn, lab in FULL_SIZE:
        if "::" + fn in test_id:
            return lab
    return None


def pytest_terminal_summary(terminalreporter):
    try:
        from tests.gpu_util import RECORDS
    except Exception:
        return
    if not RECORDS:
        return
    tw = terminalreporter
    groups = {}
    small = [0, 0, 0.0]
    for tid, name, err, kind, bound, rel, mref, over, n, ok in RECORDS:
        lab = _label(tid)
        if lab is None:
            small[0] += 1
            small[1] += 0 if ok else 1
            small[2] = max(small[2], err / bound)
            continue
        base = re.sub(r"\[.*$", "", name)
        g = groups.setdefault(lab, {})
        e = g.setdefault(base, [0.0, 0.0, 0.0, 0, 0, kind, True])
        e[0] = max(e[0], err)
        e[1] = max(e[1], rel)
        e[2] = max(e[2], mref)
        e[3] += over
        e[4] += n
        e[6] = e[6] and ok
    tw.write_line("parity vs oracle, full size (tensor: max-abs/rel-L2/max|ref|/n>2e-2; "
                  "* = derived per-element bound, ! = failed):")
    for lab, g in groups.items():
        parts = ["%s%s%s:%.1e/%.0e/%.3g/%d" % ("!" if not e[6] else "", "*" if e[5] == "derived" else "",
                                               base, e[0], e[1], e[2], e[3])
                 for base, e in g.items()]
        line = lab
        for p in parts:
            if len(line) + 1 + len(p) > 118:
                tw.write_line(line)
                line = "  "
            line += " " + p
        tw.write_line(line)
    tw.write_line("smaller cases: %d checks, %d failed, worst max-abs/bound %.2f" % tuple(small))
