"""The config selector's generated table (csrc/tgemm_choice.inc), parsed independently of
the library, and the choice it implies: used by the host tests (the selector follows the
table) and the GPU tests (every config the table names runs at full size)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def parse_choice_table():
    """The selector's generated table (csrc/tgemm_choice.inc), parsed independently."""
    text = open(os.path.join(ROOT, "tiled_dense_gemm_04_amd", "csrc", "tgemm_choice.inc")).read()
    out = {}
    for prefix in ("kF16", "kFp8"):
        ex = re.search(prefix + r"Exact\[\] = \{(.*?)\};", text, re.S).group(1)
        mo = re.search(prefix + r"Model\[\] = \{(.*?)\};", text, re.S).group(1)
        exact = [tuple(int(v) for v in m) for m in re.findall(r"\{(\d+), (\d+), (\d+), (\d+), (\d+)\}", ex)]
        model = [(int(m[0]), [float(v) for v in m[1:]])
                 for m in re.findall(r"\{(\d+), ([-\d.e+]+), ([-\d.e+]+), ([-\d.e+]+), ([-\d.e+]+)\}", mo)]
        out[prefix] = (exact, model)
    sp = re.search(r"kSplitExact\[\] = \{(.*?)\};", text, re.S).group(1)
    out["kSplit"] = [tuple(int(v) for v in m)
                     for m in re.findall(r"\{(-?\d+), (\d+), (\d+), (\d+), (-?\d+), (\d+)\}", sp) if int(m[0]) >= 0]
    return out


def expected_choice(exact, model, layout, M, N, K, tile_of, ok):
    """Exact entry for a timed shape, else the lowest predicted time over usable configs."""
    for (lay, m, n, k, cfg) in exact:
        if (lay, m, n, k) == (layout, M, N, K) and ok(cfg):
            return cfg
    best, best_us = None, None
    for cfg, (a, b, c, d) in model:
        if not ok(cfg):
            continue
        bm, bn = tile_of(cfg)
        tiles = -(-M // bm) * -(-N // bn)
        R, O, kk = -(-tiles // 256), tiles / 256, K / 1024
        us = a * R + b * R * kk + c * O + d * kk * O
        if best_us is None or us < best_us:
            best, best_us = cfg, us
    return best


def smallest_exact_shape(prefix: str, names, kind="kF16"):
    """The timed shape (A and B as given) with the fewest multiply-adds whose fastest config
    name starts with prefix, as (M, N, K, cfg), or None."""
    exact, _ = parse_choice_table()[kind]
    hits = [(M * N * K, (M, N, K, cfg)) for (lay, M, N, K, cfg) in exact
            if lay == 0 and names[cfg].startswith(prefix)]
    return min(hits)[1] if hits else None
