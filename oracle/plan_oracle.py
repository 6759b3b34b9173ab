"""Reference of the integer planning rule (bucket, pad, cost order) -- TEST
INFRASTRUCTURE ONLY, same import restrictions as ``muon_oracle``.

The pages batch matrices of similar shapes so that the Newton-Schulz recurrence
of many small matrices runs jointly and amortises kernel dispatch (DMuon
explainer on gist.science, second section 2.1, "Batching"; section 4 credits
autotuning and batching with 16% of the speed-up), and they balance work by
computational cost (DMuon abstract).  The rule below is the library's
documented contract for that step, written out plainly:

* per matrix: m = min(rows, cols), n = max(rows, cols), transposed = rows > cols
  (a square matrix is not transposed);
* precision path: "bf16" when the gradient is bf16, "f32" when it is fp32;
* tile granularity g: 64 on the f32 path; on the bf16 path 128 when m <= 128,
  else 256;
* padded dims m_pad = ceil(m / g) g and n_pad = ceil(n / g) g (zero padding);
* bucket key = (path, m_pad, n_pad): matrices of similar shape share a bucket;
* buckets are ordered by their executed cost, the sum over members of
  4 m_pad^2 n_pad + 2 m_pad^3, descending; ties keep the order in which the
  bucket key first appears;
* inside a bucket, members keep their input order (slot 0, 1, ...);
* the reported per-matrix cost is 4 m^2 n + 2 m^3 of the real shape;
* recurrence form per bucket: the Gram-space form (the iteration carried in
  the m x m Gram space, DMuon explainer on gist.science, second section 2.1
  Efficiente Gram Newton-Schulz Iteratie) on the bf16 path when n_pad > m_pad,
  m_pad >= 1024 and every member has n >= 3 m under the default option, on
  every bf16 bucket when it is forced; the short-side form otherwise, and
  always on the f32 path.  A Gram-space bucket restarts every
  ``gram_restart`` iterations (default: 2 when its padded short side is at
  most 1024, else 3); a short-side bucket reports 1.
* tuned entries (per-shape configurations measured on the device, DMuon
  explainer on gist.science, sections 2.3 and 2.4): the first entry whose
  (path, padded m, padded n) matches a bucket sets its tile (which must divide
  both padded dims; 128 or 256 on bf16, 64 on f32), its form (not the Gram
  space on f32; under the default option an entry's Gram space is refused,
  and the automatic form kept, for a bucket that the default rule keeps on
  the short side) and restart, and its XCD remap bits (default: B X only,
  bit 4).  When every bucket carries a measured per-matrix cost > 0, buckets are
  ordered by count times that cost instead of the dense cost.
"""

from __future__ import annotations

DEFAULT_GRAM_RESTART_SMALL = 2  # padded short side <= GRAM_RESTART_SMALL_MAX_M
DEFAULT_GRAM_RESTART_LARGE = 3
GRAM_RESTART_SMALL_MAX_M = 1024
GRAM_MIN_PADDED_M = 1024  # the default rule's Gram space: padded short side at least this
GRAM_MIN_ASPECT = 3       # ... and every member's long side at least this many short sides


def default_gram_restart(m_pad: int) -> int:
    return DEFAULT_GRAM_RESTART_SMALL if m_pad <= GRAM_RESTART_SMALL_MAX_M else DEFAULT_GRAM_RESTART_LARGE
DEFAULT_XCD_REMAP = 4  # bit per phase: 1 Gram, 2 square, 4 B X, 8 prod
XCD_REMAP_DEFAULT = 0xFFFFFFFF

DTYPE_F32 = 0
DTYPE_BF16 = 1


def tile_granularity(path: str, m: int) -> int:
    if path == "f32":
        return 64
    return 128 if m <= 128 else 256


def _ceil_to(x: int, g: int) -> int:
    return -(-x // g) * g


def _cost(m: int, n: int) -> int:
    return 4 * m * m * n + 2 * m * m * m


def bucket_algo(path: str, m_pad: int, n_pad: int, shapes, option: str = "auto") -> str:
    """"gram_space" or "short_side" for a bucket whose members have the real
    (m, n) in ``shapes``; option is "auto", "short_side" or "gram_space"."""
    if path != "bf16" or option == "short_side":
        return "short_side"
    if option == "gram_space":
        return "gram_space"
    if n_pad > m_pad and m_pad >= GRAM_MIN_PADDED_M and all(n >= GRAM_MIN_ASPECT * m for m, n in shapes):
        return "gram_space"
    return "short_side"


def _apply_entry(bucket, e, option_restart, option="auto", shapes=()):
    """Apply tuned entry e (dict with the library's field names and codes:
    path 0/1, algo 0 auto / 1 short side / 2 Gram space) to bucket, whose
    members have the real (m, n) in ``shapes``."""
    tile = e.get("tile", 0)
    allowed = (128, 256) if bucket["path"] == "bf16" else (64,)
    if tile and (tile not in allowed or bucket["m_pad"] % tile or bucket["n_pad"] % tile):
        raise ValueError("tile")
    forms = {0: None, 1: "short_side", 2: "gram_space"}
    if e.get("algo", 0) not in forms:
        raise ValueError("algo")
    form = forms[e.get("algo", 0)]
    if form == "gram_space" and bucket["path"] != "bf16":
        raise ValueError("gram space on f32")
    if e.get("gram_restart", 0) < 0 or e.get("cost_ms_per_matrix", 0.0) < 0:
        raise ValueError("negative")
    remap = e.get("xcd_remap", XCD_REMAP_DEFAULT)
    if remap != XCD_REMAP_DEFAULT and remap & ~0xF:
        raise ValueError("remap bits")
    if e.get("apply_pass", 0) not in (0, 1):
        raise ValueError("apply_pass")
    if tile:
        bucket["tile"] = tile
    if (form == "gram_space" and option == "auto"
            and bucket_algo(bucket["path"], bucket["m_pad"], bucket["n_pad"], shapes, "auto") != "gram_space"):
        form = None  # the default rule's accuracy guard keeps this bucket on the short side
    if form is not None:
        bucket["algo"] = form
        bucket["gram_restart"] = option_restart if form == "gram_space" else 1
    if bucket["algo"] == "gram_space" and e.get("gram_restart", 0) > 0:
        bucket["gram_restart"] = e["gram_restart"]
    if remap != XCD_REMAP_DEFAULT:
        bucket["xcd_remap"] = remap
    bucket["apply_pass"] = e.get("apply_pass", 0)
    bucket["cost"] = e.get("cost_ms_per_matrix", 0.0)


def plan_reference(descs, algo: str = "auto", gram_restart: int = 0, tuned=None):
    """descs: list of (rows, cols, grad_dtype, param_dtype) with dtype codes
    0 = fp32, 1 = bf16.  Returns a list of per-matrix dicts with keys
    bucket, slot, transposed, m, n, m_pad, n_pad, cost, and the list of
    buckets (path, m_pad, n_pad, members, algo, gram_restart) in execution
    order."""
    items = []
    keys_in_order = []
    members = {}
    for idx, (r, c, gd, _pd) in enumerate(descs):
        r, c = int(r), int(c)
        if r <= 0 or c <= 0:
            raise ValueError("matrix dims must be positive")
        m, n = min(r, c), max(r, c)
        path = "bf16" if gd == DTYPE_BF16 else "f32"
        g = tile_granularity(path, m)
        key = (path, _ceil_to(m, g), _ceil_to(n, g))
        if key not in members:
            members[key] = []
            keys_in_order.append(key)
        members[key].append(idx)
        items.append({"transposed": r > c, "m": m, "n": n, "m_pad": key[1],
                      "n_pad": key[2], "cost": _cost(m, n), "key": key})
    first_seen = {k: i for i, k in enumerate(keys_in_order)}
    info = {}
    for key in keys_in_order:
        form = bucket_algo(key[0], key[1], key[2], [(items[i]["m"], items[i]["n"]) for i in members[key]], algo)
        restart = gram_restart if gram_restart > 0 else default_gram_restart(key[1])
        bk = {"path": key[0], "m_pad": key[1], "n_pad": key[2], "members": list(members[key]),
              "algo": form, "gram_restart": restart if form == "gram_space" else 1,
              "tile": tile_granularity(key[0], key[1]), "xcd_remap": DEFAULT_XCD_REMAP, "apply_pass": 0,
              "cost": 0.0}
        code = DTYPE_BF16 if key[0] == "bf16" else DTYPE_F32
        for e in tuned or []:
            if (e["path"], e["padded_m"], e["padded_n"]) == (code, key[1], key[2]):
                _apply_entry(bk, e, restart, algo, [(items[i]["m"], items[i]["n"]) for i in members[key]])
                break
        info[key] = bk
    measured = bool(keys_in_order) and all(info[k]["cost"] > 0 for k in keys_in_order)
    if measured:
        order = sorted(keys_in_order, key=lambda k: (-len(members[k]) * info[k]["cost"], first_seen[k]))
    else:
        order = sorted(keys_in_order, key=lambda k: (-len(members[k]) * _cost(k[1], k[2]), first_seen[k]))
    buckets = []
    for b, key in enumerate(order):
        for slot, idx in enumerate(members[key]):
            items[idx]["bucket"] = b
            items[idx]["slot"] = slot
        buckets.append(info[key])
    return items, buckets
