"""Error kinds the oracle raises (test infrastructure only).

The names mirror the data errors a synchronous pack/unpack can report:
``NONFINITE`` (a weight is NaN or infinite), ``RANGE`` (a scale rounds to
infinity in binary16), ``BAD_CODE`` (a 2-bit field holds the unused pattern
0b11), ``SHAPE`` (an impossible size).
"""


class OracleError(ValueError):
    def __init__(self, kind: str, msg: str = ""):
        super().__init__(f"{kind}: {msg}" if msg else kind)
        self.kind = kind
