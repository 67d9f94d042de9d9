"""Parity figures the GPU tests measure (mask mismatch fractions, low-margin
row counts, densities).  Tests append one line each; the conftest prints them
in pytest's terminal summary, so the figures stay in the run's record even
when the tests pass quietly."""

LINES = []


def record(label, **values):
    parts = []
    for k, v in values.items():
        parts.append("%s=%s" % (k, ("%.4g" % v) if isinstance(v, float) else v))
    LINES.append("%s: %s" % (label, " ".join(parts)))
