"""Plant plausible mistakes in copies of the oracle's C source (on the CPU)
and check that at least one pin fails for each: the pins would catch a
dropped term, a wrong comparison, sign, index or operand order."""
import subprocess

import pytest

import oracle
import pins

# (name, original text, replacement) -- each original must occur exactly once
MUTANTS = [
    ("D-D case strict", "tj <= ti) vis = 1;          /* i,j in D ", "tj < ti) vis = 1;          /* i,j in D "),
    ("D-D~ case non-strict", "tj > ti) vis = 1;     /* i in D, j in D~", "tj >= ti) vis = 1;     /* i in D, j in D~"),
    ("D~-D case non-strict", "tj < ti) vis = 1;     /* i in D~, j in D", "tj <= ti) vis = 1;     /* i in D~, j in D"),
    ("D~-D~ case strict", "tj >= ti) vis = 1;   /* i,j in D~", "tj > ti) vis = 1;   /* i,j in D~"),
    ("D~ rows see future data", "tj < ti) vis = 1;     /* i in D~, j in D", "tj > ti) vis = 1;     /* i in D~, j in D"),
    ("prompt as mask kind", "col_is_data = 1; tj = 0;", "col_is_data = 0; tj = 0;"),
    ("slot index instead of label", "const int ti = tau[i % B];", "const int ti = 1 + i % B;"),
    ("rope frequency exponent", "pow(theta, -2.0 * i / d)", "pow(theta, -1.0 * i / d)"),
    ("rope sign", "v[i] = a * c - b * s;", "v[i] = a * c + b * s;"),
    ("rope physical positions", "pos[r] = (double)P + (double)(r % B);", "pos[r] = (double)P + (double)r;"),
    ("rope skips keys", "svo_rope(kd, R, Hkv, d, pos, theta);", ";"),
    ("gqa mapping", "const int kvh = h / g;", "const int kvh = h % Hkv;"),
    ("softmax scale", "scale = 1.0 / sqrt((double)d);", "scale = 1.0 / (double)d;"),
    ("unnormalised weights", "const double w = sc[j] / den;", "const double w = sc[j];"),
    ("ratio inverted", "double a = (pd > 0.0) ? pt / pd : 1.0;", "double a = (pd > 0.0) ? pd / pt : 1.0;"),
    ("target prob unnormalised", "const double pt = exp((double)z[x] - m) / s;", "const double pt = exp((double)z[x] - m);"),
    ("slot order instead of draft order", "const int k = o[r];\n            temper_row", "const int k = r - 1;\n            temper_row"),
    ("prefix off by one", "< a)) L = r - 1;", "< a)) L = r;"),
    ("assembly off by one", "ob[k] = (tb[k] <= L) ? xb[k] : -1;\n        int rs = -1;",
     "ob[k] = (tb[k] < L) ? xb[k] : -1;\n        int rs = -1;"),
    ("residual operands swapped", "const double r = pt - (double)pphi[v];", "const double r = (double)pphi[v] - pt;"),
    ("resample mass operands swapped", "double mass = use_t ? pt : pt - (double)pphi[v];", "double mass = use_t ? pt : (double)pphi[v] - pt;"),
    ("resample at wrong slot", "rs = o[L + 1];", "rs = o[L > 0 ? L : 1];"),
    ("resample fallback to the last token", "if (pick < 0) pick = last_pos;", "if (pick < 0) pick = V - 1;"),
    ("resample fallback ignores zero mass", "if (mass > 0) last_pos = v;", "last_pos = v;"),
    ("resample uses step uniform", "(double)ub[gamma], NULL", "(double)ub[0], NULL"),
    ("coupled noise subtracted", "? fmaf(l[v], inv_t, g[v]) : l[v];", "? fmaf(l[v], inv_t, -g[v]) : l[v];"),
    ("coupled ties to the largest index", "if (sc > bs) { bs = sc; best = v; }", "if (sc >= bs) { bs = sc; best = v; }"),
    ("coupled temperature multiplies", "? 1.0f / temperature : 0.f;", "? temperature : 0.f;"),
    ("coupled prefix off by one", "if ((int64_t)xb[k] != c[k]) { L = r - 1; break; }", "if ((int64_t)xb[k] != c[k]) { L = r; break; }"),
    ("coupled rejection commits the draft", "ob[o[L + 1]] = (int32_t)c[o[L + 1]];", "ob[o[L + 1]] = xb[o[L + 1]];"),
    ("coupled assembly off by one", "ob[k] = (tb[k] <= L) ? xb[k] : -1;\n        if (L < gamma)",
     "ob[k] = (tb[k] < L) ? xb[k] : -1;\n        if (L < gamma)"),
    ("route margin of the top entry only", "a = (p1 - p2 >= param) ? 1.0 : 0.0;", "a = (p1 >= param) ? 1.0 : 0.0;"),
    ("route entropy not normalised", "const double hn = (V > 1) ? h / log((double)V) : 0.0;",
     "const double hn = (V > 1) ? h : 0.0;"),
    ("route entropy sign", "a = exp(-param * hn);", "a = exp(param * hn);"),
    ("route slot order", "const float *p = probs + ((size_t)b * B + o[r]) * V;",
     "const float *p = probs + ((size_t)b * B + (r - 1)) * V;"),
    ("route sums alphas", "sum += prod;", "sum += a;"),
    ("route second entry not tracked", "else if (x > p2) p2 = x;", ";"),
    ("copies see earlier copies", "(uint8_t)(j < P || (j - P) / L == i / L);", "(uint8_t)(j < P || (j - P) / L <= i / L);"),
    ("copies indexed by position", "(uint8_t)(j < P || (j - P) / L == i / L);", "(uint8_t)(j < P || (j - P) % L == i % L);"),
    ("gather page from the row in page", "const int pg = table_row[j / page_size];", "const int pg = table_row[j % page_size];"),
    ("gather row from the page index", "j % page_size) * d, sizeof(float) * d);", "j / page_size) * d, sizeof(float) * d);"),
    ("commit skips token 0", "if (out_tokens[i] >= 0) block_tokens[i] = out_tokens[i];", "if (out_tokens[i] > 0) block_tokens[i] = out_tokens[i];"),
    ("commit fallback at R == gamma", "state[b] = (R == 0) ? 2 : (R < gamma ? 1 : 0);", "state[b] = (R == 0) ? 2 : (R <= gamma ? 1 : 0);"),
    ("commit appends unfinished blocks", "n_append[b] = (R == 0) ? B : 0;", "n_append[b] = B - R;"),
    ("append rotates at the row index", "const double pos = (double)P + (double)i;", "const double pos = (double)i;"),
    ("append leaves the length", "prefix_lens[b] = P + n;", "prefix_lens[b] = P;"),
    ("append refuses an exact fit", "if ((long long)P + n > capacity) { status[b] = 1; continue; }", "if ((long long)P + n >= capacity) { status[b] = 1; continue; }"),
    ("tree follows any earlier node", "if (pb[c] == cur && np[c] == tp[cur] && nt[c] == tt[cur]) { next = c; break; }",
     "if (pb[c] <= cur && np[c] == tp[cur] && nt[c] == tt[cur]) { next = c; break; }"),
    ("tree ignores the commit position", "if (pb[c] == cur && np[c] == tp[cur] && nt[c] == tt[cur]) { next = c; break; }",
     "if (pb[c] == cur && nt[c] == tt[cur]) { next = c; break; }"),
    ("tree compares the child's own choice", "if (pb[c] == cur && np[c] == tp[cur] && nt[c] == tt[cur]) { next = c; break; }",
     "if (pb[c] == cur && np[c] == tp[cur] && nt[c] == tt[c]) { next = c; break; }"),
    ("tree commits at the root", "commit_pos[b] = tp[cur];", "commit_pos[b] = tp[0];"),
    ("temperature multiplies", "z[v] = l[v] * inv_t;", "z[v] = l[v] / inv_t;"),
    ("temperature ignored", "z[v] = l[v] * inv_t;", "z[v] = l[v];"),
    ("resample row untempered", "ob[rs] = (int32_t)svo_residual(z, pk,",
     "ob[rs] = (int32_t)svo_residual(logits + ((size_t)b * B + rs) * V, pk,"),
    ("coupled verifies every slot", "if (tb[k] > gamma) continue;   /* not verified in this call */", ";"),
    ("confidence without the max shift", "for (int64_t v = 0; v < V; ++v) s += exp((double)l[v] - m);\n    return 1.0 / s;",
     "for (int64_t v = 0; v < V; ++v) s += exp((double)l[v]);\n    return 1.0 / s;"),
    ("confidence as the sum", "for (int64_t v = 0; v < V; ++v) s += exp((double)l[v] - m);\n    return 1.0 / s;",
     "for (int64_t v = 0; v < V; ++v) s += exp((double)l[v] - m);\n    return s;"),
    ("threshold not strict", "if (c > (double)threshold) {", "if (c >= (double)threshold) {"),
    ("confidence ties to the larger slot", "if (best < 0 || c > bc) { best = s; bc = c; }",
     "if (best < 0 || c >= bc) { best = s; bc = c; }"),
    ("lowest confidence first", "if (best < 0 || c > bc) { best = s; bc = c; }",
     "if (best < 0 || c < bc) { best = s; bc = c; }"),
    ("decided slots compete", "if (state[s] >= 0) continue;\n        const double c", ";\n        const double c"),
    ("no fallback commit", "if (n == 0 && best >= 0) {", "if (0) {"),
    ("walk leaves finished blocks", "if (!open) break;", ";"),
    ("walk compares positions only", "eq = (z[s] == (cm[s] >= 0 ? cm[s] : y[s]));",
     "eq = ((z[s] >= 0) == ((cm[s] >= 0 ? cm[s] : y[s]) >= 0));"),
    ("walk ignores the commit", "eq = (z[s] == (cm[s] >= 0 ? cm[s] : y[s]));", "eq = (z[s] == y[s] || cm[s] >= 0);"),
    ("walk takes any later node", "if (pb[c] != cur) continue;\n                const int32_t *z", "if (pb[c] < cur) continue;\n                const int32_t *z"),
    ("next state from the root", "const int32_t *y = sb + (size_t)cur * L, *cm = cb + (size_t)cur * L;\n        for (int s = 0; s < L; ++s) next_state",
     "const int32_t *y = sb, *cm = cb;\n        for (int s = 0; s < L; ++s) next_state"),
    ("state tree ignores the temperature", "const float inv_t = temperature > 0.f ? 1.0f / temperature : 0.0f;\n#pragma omp parallel for schedule(dynamic, 1) collapse(2)",
     "const float inv_t = 0.0f;\n#pragma omp parallel for schedule(dynamic, 1) collapse(2)"),
]


@pytest.fixture(scope="module")
def src_text():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, src_text, name, old, new):
    assert src_text.count(old) == 1, f"mutation site not unique/present: {old!r}"
    mut = src_text.replace(old, new)
    src = tmp_path / "svo_mut.c"
    src.write_text(mut)
    lib = str(tmp_path / "libsvo_mut.so")
    subprocess.run(oracle.gcc_cmd(str(src), lib), check=True)
    o = oracle.Oracle(lib)
    try:
        pins.all_pins(o)
    except (AssertionError, oracle.OracleError, IndexError, ValueError):
        return
    pytest.fail(f"no pin caught mutant '{name}'")


def test_unmutated_passes_all_pins():
    pins.all_pins(oracle.Oracle())
