"""Reader for the small ``key = value`` text fixtures in this folder."""

from pathlib import Path

HERE = Path(__file__).resolve().parent


def load(name: str) -> dict:
    out = {}
    for line in (HERE / name).read_text(encoding="utf-8").splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, val = line.partition("=")
        out[key.strip()] = val.strip()
    return out
