"""CPU fp64 oracle (test infrastructure only; see pa_oracle's header).

``oracle.X`` resolves to ``oracle.pa_oracle.X`` at call time, so a test that
plants a mistake in pa_oracle sees it through this package too.
"""
from . import pa_oracle


def __getattr__(name):
    return getattr(pa_oracle, name)
