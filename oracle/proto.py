"""LL and LL128 line codecs (test infrastructure only).

"Collective communication: NCCL's algorithms and protocols, and custom
all-reduce", section "Protocols" (its table of the three transports):

* LL line: 4 payload bytes + a 4-byte flag, 8 bytes in all; the reader spins
  on the flag; half of the bytes moved are payload.
* LL128 line: 120 payload bytes + an 8-byte flag, 128 bytes in all; 15/16 of
  the bytes moved are payload (the page rounds this to 94 %).
* Simple: a whole block is written, fenced, then signalled by one flag;
  practically every byte moved is payload.

The pages give only the byte counts.  Layout taken (little-endian):
LL line = payload bytes 0-3, flag (uint32) bytes 4-7; LL128 line = payload
bytes 0-119, flag (uint64) bytes 120-127.  The payload byte stream fills the
lines in order and the last line is zero-padded.  A flag of 0 is never used,
so zeroed memory never looks like an arrived line.
"""

import numpy as np

LL_LINE, LL_DATA = 8, 4
LL128_LINE, LL128_DATA = 128, 120


def _lines(nbytes: int, data: int) -> int:
    return -(-nbytes // data)


def ll_lines(nbytes: int) -> int:
    return _lines(nbytes, LL_DATA)


def ll128_lines(nbytes: int) -> int:
    return _lines(nbytes, LL128_DATA)


def wire_bytes(nbytes: int, proto: str) -> int:
    """Bytes that carry an `nbytes` payload under `proto`."""
    if proto == "simple":
        return nbytes
    if proto == "ll":
        return LL_LINE * ll_lines(nbytes)
    if proto == "ll128":
        return LL128_LINE * ll128_lines(nbytes)
    raise ValueError(f"unknown protocol {proto!r}")


def _pack(payload, flag, data, line, flag_dtype):
    if flag == 0:
        raise ValueError("flag 0 is reserved for 'nothing arrived'")
    p = np.frombuffer(np.ascontiguousarray(payload).tobytes(), dtype=np.uint8)
    n = _lines(len(p), data)
    out = np.zeros((n, line), dtype=np.uint8)
    padded = np.zeros(n * data, dtype=np.uint8)
    padded[: len(p)] = p
    out[:, :data] = padded.reshape(n, data)
    out[:, data:] = np.frombuffer(
        np.array([flag] * n, dtype=flag_dtype).tobytes(), dtype=np.uint8
    ).reshape(n, line - data)
    return out.reshape(-1)


def _unpack(lines, flag, nbytes, data, line, flag_dtype):
    b = np.asarray(lines, dtype=np.uint8).reshape(-1, line)
    flags = np.frombuffer(b[:, data:].tobytes(), dtype=flag_dtype)
    if not np.all(flags == flag_dtype(flag)):
        bad = int(np.argmax(flags != flag_dtype(flag)))
        raise ValueError(f"line {bad} has not arrived (flag {int(flags[bad])} != {flag})")
    return b[:, :data].reshape(-1)[:nbytes].copy()


def ll_pack(payload, flag: int) -> np.ndarray:
    """Payload bytes -> LL lines (uint8), each {4 B data, 4 B flag}."""
    return _pack(payload, flag, LL_DATA, LL_LINE, np.uint32)


def ll_unpack(lines, flag: int, nbytes: int) -> np.ndarray:
    """LL lines -> the first `nbytes` payload bytes; every flag must match."""
    return _unpack(lines, flag, nbytes, LL_DATA, LL_LINE, np.uint32)


def ll128_pack(payload, flag: int) -> np.ndarray:
    """Payload bytes -> LL128 lines (uint8), each {120 B data, 8 B flag}."""
    return _pack(payload, flag, LL128_DATA, LL128_LINE, np.uint64)


def ll128_unpack(lines, flag: int, nbytes: int) -> np.ndarray:
    return _unpack(lines, flag, nbytes, LL128_DATA, LL128_LINE, np.uint64)


def efficiency(nbytes: int, proto: str) -> float:
    """Payload bytes / wire bytes."""
    return nbytes / wire_bytes(nbytes, proto)
