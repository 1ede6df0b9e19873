"""The pins must be strong enough to catch plausible mistakes in the oracle.

Each case copies oracle.c to a temporary directory, plants one mistake there
(a dropped term, a wrong sign, index or operand, an off-by-one), compiles it
with gcc and checks that at least one pin of ``test_oracle_pins`` rejects it.
The real oracle is never modified.
"""
import os
import shutil

import numpy as np
import pytest

import oracle
import test_oracle_pins as P

MUTANTS = {
    "bias_not_scaled": ("fabs(den + bias * floor_)", "fabs(den + bias)"),
    "readout_wrong_index": ("Sb[(size_t)r * dvb + c] * qb[r]", "Sb[(size_t)r * dvb + c] * qb[c % dqkb]"),
    "dropped_m_in_decay": ("exp(lf + *m - m_new)", "exp(lf - m_new)"),
    "normaliser_drops_i": ("n[r] = fdec * n[r] + iw * k[r]", "n[r] = fdec * n[r] + k[r]"),
    "logsigmoid_neg_branch": ("return x - log1p(exp(x));", "return -log1p(exp(x));"),
    "den_uses_k": ("den += n[r] * q[r]", "den += n[r] * k[r]"),
    "transposed_write": ("iw * kb[r] * vb[c]", "iw * kb[c % dqkb] * vb[r % dvb]"),
    "stabiliser_offset": ("fmax(lf + *m, li) + shift", "fmax(lf + *m, li) + shift + 0.25"),
    "o_gate_no_sigmoid": ("sigmoid(o_pre[(size_t)b * dvb + c])", "o_pre[(size_t)b * dvb + c]"),
    "clamp_at_one": ("floor_ = exp(-m_new)", "floor_ = 1.0"),
    "retention_gamma_on_write": ("g * S[(size_t)r * dv + c] + kt[r] * vt[c]",
                                 "S[(size_t)r * dv + c] + g * kt[r] * vt[c]"),
    "retention_gamma_index": ("1.0 - ldexp(1.0, -5 - hd)", "1.0 - ldexp(1.0, -4 - hd)"),
    "block_rows_from_wrong_block": ("const double* qb = q + (size_t)b * dqkb;", "const double* qb = q;"),
}


def _pins_pass(lib):
    """Runs a compact set of pins against ``lib``; True if all of them pass."""
    rng = P.RNG(123)
    B, H, T, dqk, dv, nb = 2, 4, 40, 8, 12, 2
    q, k, v, ip, fp, op, bs = P._inputs(rng, B, H, T, dqk, dv)
    st = P._state(rng, B, H, dqk, dv, nb)
    ok = True
    try:
        h, C, n, m = oracle.mlstm_fwd(q, k, v, ip, fp, op, bs, *st, num_blocks=nb, lib=lib)
        hb, Cb, nbf, mb = P.brute_force(q, k, v, ip, fp, op, bs, nb, *st)
        ok &= P._relerr(h, hb) < 1e-12 and np.max(np.abs(m - mb)) < 1e-12
        ok &= P._relerr(C, Cb) < 1e-12 and P._relerr(n, nbf) < 1e-12
        hd = P.direct_unstabilised(q, k, v, ip, fp, op, bs, nb, *st)
        ok &= P._relerr(h, hd) < 1e-11
        qr, kr, vr = (rng.standard_normal((1, 4, 20, 5)) for _ in range(3))
        out, S = oracle.retention_fwd(qr, kr, vr, lib=lib)
        g = P._gammas_golden()
        t = np.arange(20)
        for hh in range(4):
            D = np.where(t[:, None] >= t[None, :], g[hh] ** (t[:, None] - t[None, :]).astype(float), 0.0)
            ref = ((qr[0, hh] @ kr[0, hh].T) * D) @ vr[0, hh]
            ok &= P._relerr(out[0, hh], ref) < 1e-12
    except (ValueError, FloatingPointError):
        return False
    return bool(ok)


@pytest.fixture(scope="module")
def gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")


def test_unmodified_oracle_passes_compact_pins():
    assert _pins_pass(oracle._load())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, gcc):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation site not found: %r" % old
    mdir = tmp_path / "oracle_mutant"
    mdir.mkdir()
    (mdir / "oracle.c").write_text(src.replace(old, new))
    out = str(mdir / "liboracle_mutant.so")
    import subprocess
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    str(mdir / "oracle.c"), "-o", out, "-lm"], check=True)
    lib = oracle._load(out)
    assert not _pins_pass(lib), "planted mistake %s was not caught by the pins" % name
