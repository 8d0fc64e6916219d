"""Runs a pin module's tests as plain functions, every parameter set of their
parametrize marks included, and names the pins that fail: the harness of the
oracle mutation tests (a mistake planted in an oracle must fail a pin)."""

import itertools
import warnings


def pin_calls(module):
    """(name, function, kwargs) for every pin of `module` and parameter set."""
    for name, fn in sorted(vars(module).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        grids = []
        for m in getattr(fn, "pytestmark", []):
            if m.name != "parametrize":
                continue
            names = m.args[0]
            names = [a.strip() for a in names.split(",")] if isinstance(names, str) else list(names)
            grids.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in m.args[1]])
        for combo in itertools.product(*grids):
            kw = {}
            for c in combo:
                kw.update(c)
            yield name, fn, kw


def failing_pins(module):
    """Names of the pins of `module` that fail (an assertion, or the mutated
    oracle breaking outright)."""
    failed = []
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for name, fn, kw in pin_calls(module):
            try:
                fn(**kw)
            except Exception:
                failed.append(name)
    return failed
