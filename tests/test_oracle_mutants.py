"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, a wrong or transposed index), compiles it on the CPU and
runs the pin suite against it in a subprocess; the suite must fail. The
committed oracle itself is never modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "etp_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_sh_cg.py"),
        os.path.join(ROOT, "tests", "test_oracle_conv.py")]
# the pin files of the layers outside the convolution, by mutant name prefix
EXTRA_PINS = {"mix_": "test_oracle_mix.py", "forces_": "test_oracle_forces.py",
              "nl_": "test_oracle_neighbors.py", "np_": "test_oracle_node_product.py"}

# (name, exact text in the oracle, replacement)
MUTANTS = [
    ("racah_sign", "s += ((k & 1) ? -1.0 : 1.0) / den;", "s += ((k & 1) ? 1.0 : 1.0) / den;"),
    ("basis_sign", "U[r * d + (k + l)] = -I * ((k & 1) ? -1.0 : 1.0) * h;",
     "U[r * d + (k + l)] = I * ((k & 1) ? -1.0 : 1.0) * h;"),
    ("re_im_swap", "double keep = odd ? cimag(s) : creal(s);", "double keep = odd ? creal(s) : cimag(s);"),
    ("legendre_coef", "hd_scale(Q[l - 2][m], l + m - 1.0)", "hd_scale(Q[l - 2][m], l + m + 0.0)"),
    ("sh_sin_cos", "t = hd_scale(Sm[am], sqrt(2.0));", "t = hd_scale(Cm[am], sqrt(2.0));"),
    ("sh_norm", "double norm = sqrt((2.0 * l + 1.0) * factorial(l - am) / factorial(l + am));",
     "double norm = sqrt((2.0 * l + 1.0) * factorial(l - am) / factorial(l + am + 1));"),
    ("fwd_x_index", "oi[en.c * C + u] += we[p * C + u] * en.C * Y[en.b] * xj[en.a * C + u];",
     "oi[en.c * C + u] += we[p * C + u] * en.C * Y[en.a] * xj[en.b * C + u];"),
    ("fwd_weight_path", "oi[en.c * C + u] += we[p * C + u] * en.C * Y[en.b] * xj[en.a * C + u];",
     "oi[en.c * C + u] += we[(P - 1 - p) * C + u] * en.C * Y[en.b] * xj[en.a * C + u];"),
    ("out_offset", "en.c = t->off[p] + l3 + t->m[3 * k + 2];", "en.c = t->off[p] + l3 - t->m[3 * k + 2];"),
    ("vjp_gx_drop_C", "gxj[en.a * C + u] += wv * en.C * Y[en.b] * g;", "gxj[en.a * C + u] += wv * Y[en.b] * g;"),
    ("vjp_Z_drop_w", "Z[en.b] += en.C * wv * xa * g;", "Z[en.b] += en.C * xa * g;"),
    ("vjp2_dG_drop_Yd", "en.C * (Y[en.b] * (wv * Xa + Wv * xa) + Yd[en.b] * wv * xa);",
     "en.C * (Y[en.b] * (wv * Xa + Wv * xa));"),
    ("vjp2_dr_drop_H", "s += Z1[b] * dY[kd * Dsh + b] + Z2[b] * HV[kd * Dsh + b];",
     "s += Z1[b] * dY[kd * Dsh + b];"),
    ("vjp2_dx_swap", "dxj[en.a * C + u] += en.C * g * (Y[en.b] * Wv + Yd[en.b] * wv);",
     "dxj[en.a * C + u] += en.C * g * (Y[en.b] * wv + Yd[en.b] * Wv);"),
    ("hyperdual_mixed", "x.a * y.d + x.b * y.c + x.c * y.b + x.d * y.a};", "x.a * y.d + x.b * y.c + x.d * y.a};"),
    ("mix_rank", "rank[p] = count[l3]++;", "rank[p] = count[l3];"),
    ("mix_transposed_W", "yr[v] += Wl[(int64_t)u * C + v] * o[u];", "yr[v] += Wl[(int64_t)v * C + u] * o[u];"),
    ("mix_wgrad_transposed", "G[(int64_t)u * C + v] += o[u] * gyr[v];", "G[(int64_t)v * C + u] += o[u] * gyr[v];"),
    ("mix_wgrad_component", "const double *gyr = gy + ((int64_t)i * Dy + l * l + mi) * C;",
     "const double *gyr = gy + ((int64_t)i * Dy + l * l + (2 * l - mi)) * C;"),
    ("forces_sign", "F[3 * (int64_t)src[e] + c] -= gr[3 * e + c];", "F[3 * (int64_t)src[e] + c] += gr[3 * e + c];"),
    ("forces_dst_index", "F[3 * i + c] += gr[3 * e + c];", "F[3 * (int64_t)src[e] + c] += gr[3 * e + c];"),
    ("nl_not_strict", "if (r2 < rc2) {", "if (r2 <= rc2) {"),
    ("nl_no_min_image", "d[c] = fmaf(-box[c], rintf(dc / box[c]), dc);", "d[c] = dc;"),
    ("nl_floor_image", "d[c] = fmaf(-box[c], rintf(dc / box[c]), dc);",
     "d[c] = fmaf(-box[c], floorf(dc / box[c]), dc);"),
    ("nl_vec_sign", "const float dc = or_wrap(pos[3 * j + c], box[c]) - qi[c];",
     "const float dc = qi[c] - or_wrap(pos[3 * j + c], box[c]);"),
    ("nl_self", "if (j == i)\n            continue;", "if (j == i && i < 0)\n            continue;"),
    ("nl_no_wrap", "qi[c] = or_wrap(pos[3 * i + c], box[c]);", "qi[c] = pos[3 * i + c];"),
    ("np_wgrad_drop_B", "gWp[u] += t.val[q] * adj[s3 * C + u] * Bk[s1 * C + u] * Ai[s2 * C + u];",
     "gWp[u] += t.val[q] * adj[s3 * C + u] * Ai[s1 * C + u] * Ai[s2 * C + u];"),
    ("np_wgrad_step", "double *gWp = gW + ((int64_t)(k - 1) * P + p) * C;",
     "double *gWp = gW + ((int64_t)(nu - 1 - k) * P + p) * C;"),
    ("np_weight_step", "const double *Wp = W + ((int64_t)(k - 1) * P + p) * C;",
     "const double *Wp = W + ((int64_t)(nu - 1 - k) * P + p) * C;"),
    ("np_operands_swapped", "NB[r3 * C + u] += Wp[u] * t.val[q] * B[r1 * C + u] * Ai[r2 * C + u];",
     "NB[r3 * C + u] += Wp[u] * t.val[q] * Ai[r1 * C + u] * B[r2 * C + u];"),
    ("np_square_of_B", "NB[r3 * C + u] += Wp[u] * t.val[q] * B[r1 * C + u] * Ai[r2 * C + u];",
     "NB[r3 * C + u] += Wp[u] * t.val[q] * B[r1 * C + u] * B[r2 * C + u];"),
    ("np_last_only", "                oi[q] += NB[q];", "                oi[q] = NB[q];"),
    ("np_m3_sign", "const int r3 = l3 * l3 + l3 + t.m[3 * q + 2];", "const int r3 = l3 * l3 + l3 - t.m[3 * q + 2];"),
    ("np_vjp_no_out_term", "                nbb[q] = Gi[q];", "                nbb[q] = 0.0;"),
    ("np_vjp_gA_operand", "                        gi[s2 * C + u] += s * Bk[s1 * C + u];",
     "                        gi[s2 * C + u] += s * Ai[s1 * C + u];"),
    ("np_vjp_no_identity", "            gi[q] += bb[q];", "            gi[q] += 0.0 * bb[q];"),
    ("mix_vjp_transposed", "acc += Wl[(int64_t)u * C + v] * gr[v];", "acc += Wl[(int64_t)v * C + u] * gr[v];"),
    ("transpose_unstable", "int64_t k = cursor[src[e]]++;", "int64_t k = src_ptr[src[e] + 1] - 1 - (cursor[src[e]]++ - src_ptr[src[e]]);"),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                           str(mutated), "-o", str(lib), "-lm"])
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    pins = [os.path.join(ROOT, "tests", f) for k, f in EXTRA_PINS.items() if name.startswith(k)] or PINS
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *pins], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pin suite:\n{r.stdout[-2000:]}"
