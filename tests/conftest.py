"""Shared test plumbing: the `gpu` marker, golden-fixture loading, device checks."""

import os

import pytest

GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse a `key: values` fixture file (comments start with '#')."""
    out = {}
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            toks = val.split()
            vals = []
            for t in toks:
                if ":" in t:
                    vals.append(tuple(int(x) for x in t.split(":")))
                else:
                    try:
                        vals.append(int(t))
                    except ValueError:
                        vals.append(float(t))
            out[key.strip()] = vals
    return out


@pytest.fixture
def golden():
    return load_golden
