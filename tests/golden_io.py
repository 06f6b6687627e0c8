"""Reader for the hand-worked fixtures in tests/golden/: '#' comments, cases split by '---',
one 'key: values' line per field (whitespace-separated numbers)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> list[dict]:
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line == "---":
                if cur:
                    cases.append(cur)
                cur = {}
                continue
            key, vals = line.split(":", 1)
            cur[key.strip()] = [float(v) for v in vals.split()]
    if cur:
        cases.append(cur)
    return cases
