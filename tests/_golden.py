"""Reader for the hand-derived text fixtures under tests/golden."""
import os

_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    """``key value value ...`` lines -> {key: [values...]} (repeated keys -> list of lists)."""
    out = {}
    rows = []
    with open(os.path.join(_DIR, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            rows.append(parts)
            out.setdefault(parts[0], []).append(parts[1:])
    return out, rows
