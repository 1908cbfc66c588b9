"""Measured parity errors of the running test, printed by conftest after the test's call phase
(pytest captures the test's own output while it runs)."""

PENDING: list[str] = []


def report(eo: float, ef: float) -> None:
    PENDING.append(f"[err] rel L2 o={eo:.3e} final={ef:.3e}")


def report_named(**errs: float) -> None:
    PENDING.append("[err] rel L2 " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
