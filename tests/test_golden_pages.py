"""Figures the SPECTRE article prints, checked against this build.

The article prints no worked numeric example of the mix itself; what it does
print is a memory estimate for the complex spectra and the fraction of bins a
truncated model keeps.  These are consistency checks of the build's sizes
against the article's figures (the workspace formula, the truncated
workload's keep_bins), not pins of the mix's arithmetic: the oracle's pins are
in test_oracle_pins.py and test_oracle_mutants.py.
"""
import json
import os

import efficient_attention_fft_amd as sm
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
FIG = json.load(open(os.path.join(HERE, "golden", "page_figures.json")))


def test_spectrum_workspace_matches_article_memory_estimate():
    """Sanity check of the workspace formula (no arithmetic of the mix is
    involved): one tensor's spectrum in the workspace (binary32 half
    spectrum: L/2 complex bins per channel = 4 bytes per real element) has
    the size the article gives for the half-precision full spectrum of the
    same shape, the two encodings happening to cost the same.
    L = 131072 plans as 64 x 2 x 1024: the first pass writes the spectra of
    q, k and v, the second pass writes them again (out of place, in the LDS
    pass's layout), so the workspace holds six spectra plus the gate table."""
    f = FIG["complex_intermediate"]
    st, plan = sm.spectre_mix_plan(f["L"])
    assert st == sm.SPECTRE_OK and plan == (64, 2, 1024)
    ws = sm.spectre_mix_workspace_bytes(f["B"], f["H"], f["L"], f["D"], sm.SPECTRE_F32)
    gate_table = 4 * f["H"] * f["L"]  # the B pass's gate table, the rest of the workspace
    assert ws - gate_table == 6 * f["bytes"]
    assert f["bytes"] == 256 * 2 ** 20


def test_truncated_workload_keeps_the_articles_lower_fraction():
    """The band-truncated workload keeps the same share of the half spectrum
    as the article's lower retention figure (1024 of the 4097 bins of an
    8192-token sequence)."""
    f = FIG["truncation_retention"]
    nb_page = f["L"] // 2 + 1
    assert abs(f["kept_low"] / nb_page - f["fraction_low"]) < 1e-3
    assert abs(f["kept_high"] / nb_page - f["fraction_high"]) < 1e-3
    w = workloads.WORKLOADS[4]
    assert abs(w.keep_bins / w.nbins - f["fraction_low"]) < 1e-3
    # keep_bins counts the DC bin: floor(fraction * L / 2) + 1
    assert w.keep_bins == int(f["fraction_low"] * w.L / 2) + 1
