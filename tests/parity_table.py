"""Format the PARITY records of the full-size GPU parity tests as a table.

Usage: python tests/parity_table.py PARITY_JSONL > table.md
(the records come from ``SD_PARITY_LOG=PARITY_JSONL pytest
tests/test_gpu_fullsize.py -m gpu``).
"""
import json
import sys

COLS = [
    ("workload", "workload"), ("requests", "requests"), ("rows", "draft rows"),
    ("attn_max_abs", "attn max-abs"), ("attn_rel_l2", "attn rel-L2"),
    ("prob_max_abs", "prob max-abs"),
    ("draft_token_near_ties", "draft-token near-ties (Gumbel gap)"),
    ("draft_token_mismatch", "draft-token mismatches"),
    ("staged_near_accept", "staged: accept near-ties"),
    ("staged_near_sample", "staged: draw near-ties"),
    ("staged_mismatch", "staged: mismatches"),
    ("e2e_near_accept", "end-to-end: accept near-ties"),
    ("e2e_near_sample", "end-to-end: draw near-ties"),
    ("e2e_excused", "end-to-end: excused requests"),
    ("e2e_mismatch", "end-to-end: mismatches"),
    ("mean_accepted", "mean accepted"),
]


def fmt(v):
    if isinstance(v, float):
        return f"{v:.3g}"
    return str(v)


def main(path):
    recs = [json.loads(l) for l in open(path) if l.strip()]
    print("| " + " | ".join(h for _, h in COLS) + " |")
    print("|" + "---|" * len(COLS))
    for r in recs:
        print("| " + " | ".join(fmt(r.get(k, "")) for k, _ in COLS) + " |")


if __name__ == "__main__":
    main(sys.argv[1])
