"""Lines the GPU tests want in the run's final summary (printed by the
terminal-summary hook in conftest.py, so they appear even under -q): the
rows checked by each full-size comparison and the elements the fp32
cancellation allowance admitted."""
LINES = []
ADMITTED = {}


def line(msg: str):
    LINES.append(msg)


def admitted(case: str, n: int, elements: int):
    ADMITTED[case] = (int(n), int(elements))


def summary():
    out = list(LINES)
    if ADMITTED:
        nz = {k: v for k, v in ADMITTED.items() if v[0]}
        out.append(f"fp32 cancellation allowance: 0 elements admitted in "
                   f"{len(ADMITTED) - len(nz)} of {len(ADMITTED)} recorded cases")
        for k, (n, e) in sorted(nz.items()):
            out.append(f"  {k}: {n} of {e} elements admitted")
    return out
