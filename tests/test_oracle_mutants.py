"""The oracle's pins must fail a wrong oracle (no GPU).

Each case plants one plausible mistake in a copy of ``oracle/oracle.c``,
builds it with gcc the way ``oracle.build`` does, and runs the oracle's own
CPU pin tests against it in a child process (``ORACLE_LIB`` selects the
build).  A pin set that passed a mutant would not be pinning the oracle.  The
unmodified source, built and run the same way, must pass the same tests, so a
failure is the mutant's and not the harness's.

The mistakes, and the passages the pins that catch them follow:

- chunk ranges without the first_page_offset shift (PR #984 body items 2
  and 4), in the partial and in the MLA chunk mode;
- the flat gather without the first_page_offset shift (the CSR view,
  Issue #898 item 1);
- query head h reading KV head h % Hkv instead of h / G (GQA grouping);
- scores without sm_scale;
- the LSE in natural-log units instead of log2 (base-2 scores, PR #984 body
  item 2);
- the merge weighting rows by e^(lse - m) instead of 2^(lse - m) (the
  closed-form rescale, Issue #898 item 3);
- the MLA score without its second key stream (sparse paged decode doc, the
  DSA section);
- the plan keeping the smallest qualifying pages-per-chunk instead of the
  largest (PR #984 body item 4).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

PARTIAL_RANGE = ("            tb = t * span - j->fpo[r];\n            te = (t + 1) * span - j->fpo[r];",
                 "            tb = t * span;\n            te = (t + 1) * span;")

# name: (old text, new text, which occurrence of old (0-based), pin test files)
MUTANTS = {
    "partial_range_no_fpo": PARTIAL_RANGE + (0, ["test_oracle_chunks.py"]),
    "mla_range_no_fpo": PARTIAL_RANGE + (1, ["test_oracle_chunks.py"]),
    "gather_no_fpo": ("        int64_t slot = j->fpo[r] + tok_begin + i;",
                      "        int64_t slot = tok_begin + i;", 0,
                      ["test_oracle_attention.py", "test_oracle_chunks.py"]),
    "gqa_interleaved": ("    const int32_t kvh = h / group;              /* query head h reads KV head h / group */",
                        "    const int32_t kvh = h % j->hkv;", 0,
                        ["test_oracle_attention.py"]),
    "score_no_scale": ("        s[i] = j->sm_scale * dot;", "        s[i] = dot;", 0,
                       ["test_oracle_attention.py"]),
    "lse_natural_log": ("    *lse2 = (m + log(z)) / log(2.0);", "    *lse2 = m + log(z);", 0,
                        ["test_oracle_attention.py"]),
    "merge_natural_exp": ("                double w = pow(2.0, l - m);",
                          "                double w = exp(l - m);", 0,
                          ["test_oracle_attention.py"]),
    "mla_no_second_stream": ("        s[i] = j->sm_scale * dot + j->sm_scale * dot_x;",
                             "        s[i] = j->sm_scale * dot;", 0, ["test_oracle_mla.py"]),
    "plan_smallest_c": ("            if (n * wg_per_chunk >= target) best = c;   /* keep the largest */",
                        "            if (n * wg_per_chunk >= target && best < 0) best = c;", 0,
                        ["test_oracle_csr_plan.py"]),
}


def _build(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, "lib" + name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", so, c, "-lm",
                           "-lpthread"])
    return so


def _run_pins(lib, files):
    env = dict(os.environ, ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + \
        [os.path.join(ROOT, "tests", f) for f in files]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _mutate(name):
    old, new, which, _ = MUTANTS[name]
    text = open(SRC).read()
    pos = -1
    for _ in range(which + 1):
        pos = text.index(old, pos + 1)
    return text[:pos] + new + text[pos + len(old):]


@pytest.fixture(scope="module")
def control_lib(tmp_path_factory):
    return _build(open(SRC).read(), str(tmp_path_factory.mktemp("orc_control")), "control")


@pytest.mark.parametrize("files", sorted({tuple(m[3]) for m in MUTANTS.values()}))
def test_unmodified_oracle_passes_its_pins(control_lib, files):
    r = _run_pins(control_lib, list(files))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_fail_a_planted_mistake(tmp_path, name):
    lib = _build(_mutate(name), str(tmp_path), name)
    r = _run_pins(lib, MUTANTS[name][3])
    # pytest exits 1 when tests ran and some failed (not 2-5: errors, no tests)
    assert r.returncode == 1 and " failed" in r.stdout, \
        "mutant %s passed its pins:\n%s" % (name, r.stdout[-3000:])
