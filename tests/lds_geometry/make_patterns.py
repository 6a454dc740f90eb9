"""Writes the address patterns that lds_probe.hip times.

Three families, for each access (ds_read_b32 / b64 / b128, ds_write_b128):

* ``full_lin``: all 64 lanes at consecutive addresses (the throughput base).
* ``pair_same_i_j`` / ``pair_diff_i_j``: only lanes i and j active; lane i
  at byte 0, lane j at byte 4096 (same bank, another word, for any bank line
  that divides 4096) or at 4096 + 16 (another bank).  A slower "same" than
  "diff" means the hardware services lanes i and j in the same phase.
* ``line_X``: lanes 0 and 1 active at bytes 0 and X: a conflict appears
  exactly when X is a multiple of the bank-line size (banks x 4 bytes).

Plus the operand-tile patterns of the GEMM kernels (K-major tiles, 16-byte
chunks, rows of 64 or 128 bytes) under each candidate swizzle.

Usage: python make_patterns.py patterns.txt [--no-pairs | --pairs-only] [--ops=r128,w128]
"""
import sys

OPS = {"r32": 4, "r64": 8, "r128": 16, "w128": 16}
INACTIVE = -1


def _line(name, op, addrs):
    assert len(addrs) == 64
    return f"{name} {op} " + " ".join(str(a) for a in addrs)


def swz(row, chunk, row_bytes, kind):
    """Candidate LDS maps for a K-major tile (byte offset)."""
    off = row * row_bytes + 16 * chunk
    if kind == "none":
        return off
    if kind == "x8":      # 16-byte unit XOR (line index mod 8), 128-byte lines
        return off ^ (((off >> 7) & 7) << 4)
    if kind == "x16":     # 16-byte unit XOR (line index mod 16), 256-byte lines
        return off ^ (((off >> 8) & 15) << 4)
    if kind == "mix":     # chunk ^ ((row ^ row>>3) & 7), 128-byte rows only
        return row * row_bytes + 16 * (chunk ^ ((row ^ (row >> 3)) & 7))
    raise ValueError(kind)


def main(path, pairs=True, pairs_only=False, ops=None):
    out = []
    for op, w in OPS.items():
        if ops and op not in ops:
            continue
        if pairs_only:
            for i in range(64):
                for j in range(i + 1, 64):
                    a = [INACTIVE] * 64
                    a[i], a[j] = 0, 4096
                    out.append(_line(f"pair_same_{i}_{j}", op, a))
            continue
        out.append(_line(f"full_lin", op, [w * l for l in range(64)]))
        out.append(_line(f"full_bcast", op, [0] * 64))
        for X in (16, 32, 64, 128, 256, 512, 1024):
            if X % w:
                continue
            a = [INACTIVE] * 64
            a[0], a[1] = 0, X
            out.append(_line(f"line_{X}", op, a))
        for i in range(64 if pairs else 0):
            for j in range(i + 1, 64):
                for kind, aj in (("same", 4096), ("diff", 4096 + 16)):
                    a = [INACTIVE] * 64
                    a[i], a[j] = 0, aj
                    out.append(_line(f"pair_{kind}_{i}_{j}", op, a))
    if pairs_only:
        with open(path, "w") as f:
            f.write("\n".join(out) + "\n")
        print(f"{len(out)} patterns -> {path}")
        return
    # GEMM operand-tile patterns.
    for kind in ("none", "x8", "x16"):
        # A 32-byte-per-lane operand read (128-byte rows): lane l reads
        # chunks 4*kk + 2*(l/32) + h of row l%32 as two ds_read_b128 (h = 0,
        # 1).  (The MX kernels' actual order, chunk 4*kk + 2*h + l/32, is the
        # mfma32 pattern below.)
        for kk in range(2):
            for h in range(2):
                a = [swz(l % 32, 4 * kk + 2 * (l // 32) + h, 128, kind) for l in range(64)]
                out.append(_line(f"mx32_{kind}_kk{kk}_h{h}", "r128", a))
        # MN-major loader store after the register transpose: lane t owns
        # k-chunk t%8 of rows 8*(t/8) + c, written one c at a time.
        for c in range(8):
            a = [swz(8 * (l // 8) + c, l % 8, 128, kind) for l in range(64)]
            out.append(_line(f"mnstore_{kind}_c{c}", "w128", a))
    for kind in ("none", "x8", "x16", "mix"):
        for row_bytes in (64, 128, 256):
            if kind == "mix" and row_bytes != 128:
                continue
            chunks = row_bytes // 16
            # 32x32 MFMA operand: lane -> row l%32, chunk c0 + l//32.
            for c0 in range(0, chunks, 2):
                a = [swz(l % 32, c0 + l // 32, row_bytes, kind) for l in range(64)]
                out.append(_line(f"mfma32_{kind}_rb{row_bytes}_c{c0}", "r128", a))
            # 16x16 MFMA operand: lane -> row l%16, chunk c0 + l//16.
            for c0 in range(0, chunks, 4):
                if c0 + 3 >= chunks:
                    continue
                a = [swz(l % 16, c0 + l // 16, row_bytes, kind) for l in range(64)]
                out.append(_line(f"mfma16_{kind}_rb{row_bytes}_c{c0}", "r128", a))
            # Loader store: consecutive lanes take consecutive chunks of a row.
            a = [swz(l // chunks, l % chunks, row_bytes, kind) for l in range(64)]
            out.append(_line(f"store_{kind}_rb{row_bytes}", "w128", a))
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")
    print(f"{len(out)} patterns -> {path}")


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    ops = None
    for a in sys.argv[1:]:
        if a.startswith("--ops="):
            ops = a.split("=", 1)[1].split(",")
    main(args[0] if args else "patterns.txt", pairs="--no-pairs" not in sys.argv,
         pairs_only="--pairs-only" in sys.argv, ops=ops)
