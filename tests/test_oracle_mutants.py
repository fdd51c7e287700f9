"""Pin strength: plausible mistakes planted in copies of the oracle source
must each fail at least one pin of tests/oracle_pins.py.

Each mutant is a textual edit of oracle/kla_oracle.c compiled with gcc into
a temporary directory and exercised in a child process (a mutant that
crashes counts as caught).  Nothing here touches a GPU.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kla_oracle.c")

W_MARK = "    /* S = S~ + beta k e^T */\n"
O_MARK = "    /* o = S^T q */\n"


def _swap_write_and_read(src):
    """Read before the write (the pre-write readout reading)."""
    a = src.index(W_MARK)
    b = src.index(O_MARK)
    end = src.index("\n}\n", b) + 1
    write_blk, read_blk = src[a:b], src[b:end]
    return src[:a] + read_blk + write_blk + src[end:]


def _first(s, old, new):
    """Replace the first occurrence: the scalar step precedes the per-channel one."""
    return s.replace(old, new, 1)


MUTANTS = {
    "no_decay": lambda s: _first(s, "S[(size_t)i * dv + j] *= alpha;", "(void)alpha;"),
    "beta_unnormalised": lambda s: _first(s, "eta / (kk + eps)", "eta"),
    "beta_norm_not_squared": lambda s: _first(s, "eta / (kk + eps)", "eta / (__builtin_sqrt(kk) + eps)"),
    "beta_drops_eps": lambda s: _first(s, "eta / (kk + eps)", "eta / kk"),
    "beta_times_alpha": lambda s: _first(s, "eta / (kk + eps)", "alpha * eta / (kk + eps)"),
    "residual_sign": lambda s: _first(s, "e[j] -= S[(size_t)i * dv + j] * k[i];",
                                         "e[j] += S[(size_t)i * dv + j] * k[i];"),
    "residual_undecayed": lambda s: _first(s, "e[j] -= S[(size_t)i * dv + j] * k[i];",
                                              "e[j] -= S[(size_t)i * dv + j] * k[i] / alpha;"),
    "write_uses_v": lambda s: _first(s, "S[(size_t)i * dv + j] += bk * e[j];",
                                        "S[(size_t)i * dv + j] += bk * v[j];"),
    "read_with_key": lambda s: _first(s, "o[j] += S[(size_t)i * dv + j] * q[i];",
                                         "o[j] += S[(size_t)i * dv + j] * k[i];"),
    "read_before_write": _swap_write_and_read,
    "ignores_initial_state": lambda s: _first(s, "if (initial_state)\n", "if (0)\n"),
    "decode_swaps_q_and_k": lambda s: _first(s, 
        "kla_token(state + sh * sdim, e, q + sh * dk, k + sh * dk,",
        "kla_token(state + sh * sdim, e, k + sh * dk, q + sh * dk,"),
    "drops_last_token": lambda s: _first(s, "t < cu_seqlens[s + 1]; ++t", "t + 1 < cu_seqlens[s + 1]; ++t"),
    "direct_mode_ignored": lambda s: _first(s, "beta_direct ? eta : eta / (kk + eps)",
                                               "eta / (kk + eps)"),
    "missing_alpha_is_zero": lambda s: _first(s, "alpha ? alpha[th] : 1.0", "alpha ? alpha[th] : 0.0"),
    "decode_missing_alpha_is_zero": lambda s: _first(s, "alpha ? alpha[sh] : 1.0",
                                                        "alpha ? alpha[sh] : 0.0"),
    "decode_drops_direct_mode": lambda s: _first(s, "eps, beta_direct, dk, dv, o + sh * dv",
                                                    "eps, 0, dk, dv, o + sh * dv"),
    "decay_after_write": lambda s: _first(_first(
        s,
        "    for (int i = 0; i < dk; ++i)\n        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha;\n",
        ""),
        "    /* o = S^T q */\n",
        "    for (int i = 0; i < dk; ++i)\n        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha;\n    /* o = S^T q */\n"),
}

CH_DECAY = ("    /* S~ = Diag(a) S: row i (key channel i) decays by a[i] */\n"
            "    for (int i = 0; i < dk; ++i)\n"
            "        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[i];\n")
CH_WRITE = "    /* S = S~ + beta k e^T */\n    for (int i = 0; i < dk; ++i) {\n        const double bk = beta * k[i];"


def _ch_residual_before_decay(src):
    """Per-channel path: the residual reads the undecayed state."""
    a = src.index(CH_DECAY)
    src = src[:a] + src[a + len(CH_DECAY):]
    b = src.index(CH_WRITE, a)
    return src[:b] + CH_DECAY + src[b:]


MUTANTS.update({
    "ch_decays_columns": lambda s: s.replace("S[(size_t)i * dv + j] *= a[i];",
                                             "S[(size_t)i * dv + j] *= a[j];"),
    "ch_first_channel_only": lambda s: s.replace("S[(size_t)i * dv + j] *= a[i];",
                                                 "S[(size_t)i * dv + j] *= a[0];"),
    "ch_no_decay": lambda s: s.replace("S[(size_t)i * dv + j] *= a[i];", "(void)a;"),
    "ch_residual_before_decay": _ch_residual_before_decay,
    "ch_fwd_scalar_stride": lambda s: s.replace("alpha + th * dk,", "alpha + th,"),
    "ch_decode_scalar_stride": lambda s: s.replace("alpha + sh * dk, eta[sh]", "alpha + sh, eta[sh]"),
    "ch_fwd_ignores_direct": lambda s: s.replace(
        "eta[th], eps, beta_direct, dk, dv, o + th * dv);\n            }\n            if (final_state) memcpy(final_state + sh * sdim, S, sizeof(double) * sdim);\n            free(S);\n        }\n    }\n    return failed ? -1 : 0;\n}\n\n/* One decode step with the per-channel",
        "eta[th], eps, 0, dk, dv, o + th * dv);\n            }\n            if (final_state) memcpy(final_state + sh * sdim, S, sizeof(double) * sdim);\n            free(S);\n        }\n    }\n    return failed ? -1 : 0;\n}\n\n/* One decode step with the per-channel"),
    "ch_decode_drops_direct": lambda s: s.replace("alpha + sh * dk, eta[sh], eps, beta_direct",
                                                  "alpha + sh * dk, eta[sh], eps, 0"),
})

CCQ_UPDATE = ("    *n += 1.0;\n"
              "    for (int i = 0; i < dk; ++i) {\n"
              "        m[i] += k[i];\n"
              "        for (int c = 0; c < dk; ++c) P[(size_t)i * dk + c] += k[i] * k[c];\n"
              "    }\n")


def _ccq_excludes_current_key(src):
    """The covariance of the keys before t (the sums updated after the read)."""
    a = src.index(CCQ_UPDATE)
    src = src[:a] + "    const double inv0 = 1.0 / (*n + 1.0); (void)inv0;\n" + src[a + len(CCQ_UPDATE):]
    b = src.index("        qc[i] = q[i] - lambda * sq;\n    }\n", a) + len("        qc[i] = q[i] - lambda * sq;\n    }\n")
    return src[:b] + CCQ_UPDATE + src[b:]


MUTANTS.update({
    "ccq_no_mean": lambda s: s.replace("const double sq = pq * inv - (m[i] * inv) * (mq * inv);",
                                       "const double sq = pq * inv;"),
    "ccq_unbiased": lambda s: s.replace("const double inv = 1.0 / *n;",
                                        "const double inv = *n > 1.0 ? 1.0 / (*n - 1.0) : 0.0;"),
    "ccq_lambda_sign": lambda s: s.replace("qc[i] = q[i] - lambda * sq;", "qc[i] = q[i] + lambda * sq;"),
    "ccq_mean_once": lambda s: s.replace("(m[i] * inv) * (mq * inv)", "(m[i] * inv) * mq"),
    "ccq_excludes_current_key": _ccq_excludes_current_key,
    "ccq_reads_raw_query": lambda s: s.replace(
        "kla_token(S, e, qc, k + th * dk,", "kla_token(S, e, q + th * dk, k + th * dk,"),
    "ccq_decode_reads_raw_query": lambda s: s.replace(
        "kla_token(state + sh * sdim, e, qc,", "kla_token(state + sh * sdim, e, q + sh * dk,"),
    "ccq_ignores_start_sums": lambda s: s.replace("if (ccq_in)\n", "if (0)\n"),
})

MUTANTS.update({
    "bwd_drops_residual_path": lambda s: s.replace("gk[i] -= sde;", "(void)sde;"),
    "bwd_drops_step_norm_term": lambda s: s.replace("for (int i = 0; i < dk; ++i) gk[i] -= c * kt[i];",
                                                    "(void)c;"),
    "bwd_dalpha_from_new_state": lambda s: s.replace("da += dS[x] * Sp[x];", "da += dS[x] * S[x];"),
    "bwd_state_grad_undecayed": lambda s: s.replace("dS[x] *= a;", "(void)a;"),
    "bwd_residual_grad_unscaled": lambda s: s.replace("for (int j = 0; j < dv; ++j) de[j] *= b;", ""),
    "bwd_dq_from_old_state": lambda s: s.replace("acc += S[(size_t)i * dv + j] * gt[j];",
                                                 "acc += Sp[(size_t)i * dv + j] * gt[j];"),
    "bwd_deta_unnormalised": lambda s: s.replace("d_eta[th] = db / (kk + eps);", "d_eta[th] = db;"),
    "bwd_ignores_final_grad": lambda s: s.replace("if (d_final)\n", "if (0)\n"),
    "bwd_write_grad_sign": lambda s: s.replace("dS[(size_t)i * dv + j] -= kt[i] * de[j];",
                                               "dS[(size_t)i * dv + j] += kt[i] * de[j];"),
})

RUNNER = textwrap.dedent("""
    import sys, functools
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import oracle
    from oracle_pins import ALL_PINS
    fwd = functools.partial(oracle.fwd, lib_path={lib!r})
    dec = functools.partial(oracle.decode_step, lib_path={lib!r})
    failed = []
    for pin in ALL_PINS:
        try:
            pin(fwd, dec)
        except Exception as e:
            failed.append(pin.__name__)
    print("FAILED_PINS", ",".join(failed))
""")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src, "mutation did not apply"
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(csrc),
                    "-o", str(lib)], check=True)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(lib))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, OMP_NUM_THREADS="2"))
    if r.returncode != 0:
        return  # crashed: caught
    line = [l for l in r.stdout.splitlines() if l.startswith("FAILED_PINS")][0]
    failed = [x for x in line.split(" ", 1)[1].split(",") if x] if " " in line else []
    assert failed, f"mutant {name} passed every pin"
