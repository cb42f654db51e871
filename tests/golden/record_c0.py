"""Write tests/golden/c0_sequence.json: SHA-256 digests of every byte the oracle produces over
the tiny configuration's prefill / decode / block verify / rollback / tree verify / commit
sequence (tests/c0_gate.py).  Calls only the oracle and the input generator.

Re-record only for a stated reason (a change to the oracle's arithmetic that a passage of
the pages justifies, or a change of the sequence itself), and name it with --reason; the
reason is kept in the file.

  python tests/golden/record_c0.py --reason "first recording"
"""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from tests import c0_gate  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c0_sequence.json")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reason", required=True)
    args = ap.parse_args()
    rec = {"source": "the refactor gate of 'Adding a model', 'The tests a new model must pass' "
                     "(exact bytes after a prefill, a decode, a block verify, a rollback, a tree "
                     "verify and a commit), on the oracle",
           "written_by": "tests/golden/record_c0.py (oracle and input generator only)",
           "reason": args.reason,
           "seed": c0_gate.SEED, "steps": list(c0_gate.STEPS),
           "digests": c0_gate.digests(c0_gate.run_oracle())}
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(OUT)


if __name__ == "__main__":
    main()
