"""The backward pins must be strong enough to catch plausible mistakes in the
oracle's backward functions.

Each case copies oracle.c to a temporary directory, plants one mistake in
oracle_mlstm_bwd or oracle_retention_bwd (a dropped term, a wrong sign, a
wrong operand, index or block, a missing decay), compiles it with gcc and
checks that the compact backward pins reject it.  The pins compare every
gradient with central finite differences of the real (unmodified) forward
oracle, so the reference never comes from the library under test.  The real
oracle is never modified.
"""
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_bwd_pins as BP

MUTANTS = {
    # mLSTM backward
    "bwd_dz_sign_dropped": ("-sdy / den * (zt > 0 ? 1.0 : -1.0)", "-sdy / den"),
    "bwd_dq_drops_normaliser_term": ("double a = nt[d] * dz;", "double a = 0.0;"),
    "bwd_dq_reads_previous_state": ("const double* Sr = St + (size_t)b * dqkb * dvb + (size_t)r * dvb;",
                                    "const double* Sr = Sp + (size_t)b * dqkb * dvb + (size_t)r * dvb;"),
    "bwd_state_grad_uses_k": ("Gr[cc] += qt[d] * dn[b * dvb + cc];", "Gr[cc] += kt[d] * dn[b * dvb + cc];"),
    "bwd_norm_grad_uses_k": ("g[d] += qt[d] * dz;", "g[d] += kt[d] * dz;"),
    "bwd_dk_drops_norm_part": ("dk[tok * dqk + d] = iw * (Gv[d] + g[d]);", "dk[tok * dqk + d] = iw * Gv[d];"),
    "bwd_dv_key_from_wrong_block": ("* kt[b * dqkb + r];", "* kt[r];"),
    "bwd_di_drops_norm_part": ("di[tok] = iw * (kGv + kg);", "di[tok] = iw * kGv;"),
    "bwd_df_sigmoid_sign": ("df[tok] = dlf * sigmoid(-f_pre[tok]);", "df[tok] = dlf * sigmoid(f_pre[tok]);"),
    "bwd_norm_grad_not_decayed": ("for (int r = 0; r < dqk; ++r) g[r] *= fdec;",
                                  "for (int r = 0; r < dqk; ++r) g[r] *= 1.0;"),
    "bwd_dlf_drops_normaliser": ("double a = 0.0, bb = np_[d] * g[d];", "double a = 0.0, bb = 0.0;"),
    "bwd_dn_without_output_gate": ("dn[c] = o * dht[c] / den;", "dn[c] = dht[c] / den;"),
    "bwd_dbias_not_scaled": ("dbias_acc += dz * fl;", "dbias_acc += dz;"),
    "bwd_floor_ignored": ("const double dz = fabs(zt) > fl ?", "const double dz = fabs(zt) >= 0.0 ?"),
    "bwd_do_pre_missing_o": ("dht[c] * y * o * (1.0 - o)", "dht[c] * y * (1.0 - o)"),
    "bwd_decay_without_stabiliser": ("const double fdec = exp(lf + mp - mt), iw = exp(i_pre[tok] - mt);",
                                     "const double fdec = exp(lf), iw = exp(i_pre[tok] - mt);"),
    # retention backward
    "ret_bwd_dq_wrong_index": ("for (int c = 0; c < dv; ++c) a += S[(size_t)r * dv + c] * gt[c];",
                               "for (int c = 0; c < dv; ++c) a += S[(size_t)r * dv + c] * gt[r % dv];"),
    "ret_bwd_G_not_decayed": ("const double gd = t == T - 1 ? 1.0 : g;", "const double gd = 1.0;"),
    "ret_bwd_dk_uses_k": ("for (int c = 0; c < dv; ++c) a += S[(size_t)r * dv + c] * vt[c];",
                          "for (int c = 0; c < dv; ++c) a += S[(size_t)r * dv + c] * kt[c % dk];"),
    "ret_bwd_dS0_undecayed": ("dS0[bh * ssz + e] = g * S[e];", "dS0[bh * ssz + e] = S[e];"),
    "ret_bwd_G_from_k": ("S[(size_t)r * dv + c] = gd * S[(size_t)r * dv + c] + qt[r] * gt[c];",
                         "S[(size_t)r * dv + c] = gd * S[(size_t)r * dv + c] + kt[r] * gt[c];"),
}

NB = 2  # two memory blocks, so that a row taken from the wrong block shows


def _fd(x, loss, eps=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        keep = x[idx]
        x[idx] = keep + eps
        lp = loss()
        x[idx] = keep - eps
        lm = loss()
        x[idx] = keep
        g[idx] = (lp - lm) / (2 * eps)
    return g


@pytest.fixture(scope="module")
def references():
    """Finite-difference gradients of the real forward oracle for one mLSTM
    case (output gate, bias, block-diagonal initial state, the floor of the
    denominator active on some tokens and not on others, z of both signs) and
    one retention case (initial state, explicit gammas)."""
    real = oracle._load()
    a, dh = BP._case(41, 1, 2, 7, 4, 6, kscale=3.0)
    B, H, T, dqk = a["q"].shape
    dv = a["v"].shape[-1]
    a["C0"] = np.random.default_rng(42).standard_normal((B, H, NB, dqk // NB, dv // NB)) * 0.3

    def loss():
        h = oracle.mlstm_fwd(a["q"], a["k"], a["v"], a["i_pre"], a["f_pre"], a["o_pre"], a["bias"],
                             a["C0"], a["n0"], a["m0"], num_blocks=NB, lib=real)[0]
        return np.sum(dh * h)

    fd = {gname: _fd(a[name], loss) for name, gname in BP.GRAD_OF.items()}
    z = oracle.mlstm_bwd(dh=dh, num_blocks=NB, lib=real, **a)["z"]

    rng = np.random.default_rng(43)
    r = dict(q=rng.standard_normal((1, 2, 7, 3)), k=rng.standard_normal((1, 2, 7, 3)),
             v=rng.standard_normal((1, 2, 7, 4)), S0=rng.standard_normal((1, 2, 3, 4)))
    gamma = np.array([0.9, 0.7])
    do = rng.standard_normal((1, 2, 7, 4))

    def rloss():
        return np.sum(do * oracle.retention_fwd(r["q"], r["k"], r["v"], gamma, r["S0"], lib=real)[0])

    rfd = {gname: _fd(r[name], rloss) for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("S0", "dS0"))}
    return dict(a=a, dh=dh, fd=fd, z=z, r=r, gamma=gamma, do=do, rfd=rfd)


def _bwd_pins_pass(lib, ref):
    """True if every gradient of both cases matches the finite differences."""
    try:
        g = oracle.mlstm_bwd(dh=ref["dh"], num_blocks=NB, lib=lib, **ref["a"])
        ok = all(BP._relerr(g[n], ref["fd"][n]) < 1e-6 for n in ref["fd"])
        r = ref["r"]
        gr = oracle.retention_bwd(r["q"], r["k"], r["v"], ref["do"], ref["gamma"], r["S0"], lib=lib)
        ok &= all(BP._relerr(gr[n], ref["rfd"][n]) < 1e-7 for n in ref["rfd"])
    except (ValueError, FloatingPointError):
        return False
    return bool(ok)


def test_case_covers_both_floor_branches_and_signs(references):
    z = references["z"]
    assert (z > 1).any() and (z < -1).any() and (np.abs(z) < 1).any()
    assert np.min(np.abs(np.abs(z) - 1)) > 1e-3  # no token within reach of the kink


def test_unmodified_oracle_passes_backward_pins(references):
    assert _bwd_pins_pass(oracle._load(), references)


@pytest.fixture(scope="module")
def gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name, tmp_path, gcc, references):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation site not found: %r" % old
    mdir = tmp_path / "oracle_mutant"
    mdir.mkdir()
    (mdir / "oracle.c").write_text(src.replace(old, new))
    out = str(mdir / "liboracle_mutant.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    str(mdir / "oracle.c"), "-o", out, "-lm"], check=True)
    lib = oracle._load(out)
    assert not _bwd_pins_pass(lib, references), "planted mistake %s was not caught by the pins" % name
