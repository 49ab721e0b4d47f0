"""Hand-derived cases in tests/golden/ against the float64 oracle (CPU only).

Each fixture states the operation it exercises (with the page and section
that define it), the inputs, and the expected O and LSE as closed-form
expressions derived by hand from the definition; they are evaluated here
with e and log only, so no stored number comes from any implementation.
"""
import glob
import math
import os

import numpy as np
import pytest

import oracle
from workloads import MLACase

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FILES = sorted(glob.glob(os.path.join(GOLDEN, "*.txt")))
_NAMES = {"e": math.e, "log": math.log, "__builtins__": {}}


def _parse(path):
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def _rows(text, evaluate=False):
    out = []
    for row in text.split(";"):
        items = row.split("   ") if evaluate else row.split()
        out.append([eval(x, _NAMES) if evaluate else float(x) for x in items if x.strip()])
    return np.array(out, dtype=np.float64)


def _case(g):
    dl, dr = int(g["d_latent"]), int(g["d_rope"])
    D = dl + dr
    P, L, ql, H = int(g["page_size"]), int(g["kv_len"]), int(g["q_len"]), int(g["num_heads"])
    rows = _rows(g["kv_rows"]).astype(np.float32)
    n_pages = (L + P - 1) // P
    num_pages = n_pages + 2
    # reversed page order: logical page i lives in pool page num_pages-1-i
    kv = np.full((num_pages, P, D), np.nan, np.float32)
    bt = np.full((1, n_pages + 1), -1, np.int32)
    for i in range(n_pages):
        bt[0, i] = num_pages - 1 - i
    for j in range(L):
        kv[bt[0, j // P], j % P] = rows[j]
    q = _rows(g["q_rows"]).astype(np.float32).reshape(1, ql, H, D)
    return MLACase(name=os.path.basename(g["_path"]), batch=1, num_heads=H, d_latent=dl,
                   d_rope=dr, page_size=P, kv_dtype="fp32", causal=bool(int(g["causal"])),
                   sm_scale=float(g["sm_scale"]), kv_lens=np.array([L], np.int32),
                   q_lens=np.array([ql], np.int32), block_table=bt, q=q, kv=kv)


def test_fixtures_present():
    assert len(FILES) >= 3


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(p) for p in FILES])
def test_oracle_matches_hand_derived_case(path):
    g = _parse(path)
    g["_path"] = path
    case = _case(g)
    O, LSE = oracle.mla_decode_ref(case)
    want_o = _rows(g["expect_O"], evaluate=True)
    want_l = _rows(g["expect_LSE"], evaluate=True).reshape(-1)
    tol = float(g["tol"])
    got_o = O[0].reshape(-1, O.shape[-1])       # rows ordered (t, h)
    got_l = LSE[0].reshape(-1)
    assert got_o.shape == want_o.shape
    assert np.max(np.abs(got_o - want_o)) <= tol
    assert np.max(np.abs(got_l - want_l)) <= tol
