"""Hand-derived fixtures; each file states the passage it follows."""
import os

GOLDEN_DIR = os.path.dirname(os.path.abspath(__file__))


def load_mask_fixture(name):
    """Return (tau, visibility [2B][2B] as nested lists of bool) from a fixture file."""
    rows = {}
    tau = None
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, _, rest = line.partition(":")
            if head == "tau":
                tau = [int(t) for t in rest.split()]
            else:
                rows[head] = rest.split()
    B = len(tau)

    def idx(label):
        return B + int(label[2:]) if label.startswith("~D") else int(label[1:])

    vis = [[False] * (2 * B) for _ in range(2 * B)]
    for label, cols in rows.items():
        for c in cols:
            vis[idx(label)][idx(c)] = True
    assert len(rows) == 2 * B
    return tau, vis
