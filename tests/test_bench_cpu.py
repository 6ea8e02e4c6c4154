"""Host-side checks of bench.py: the committed rocprofv3 counter summaries
must be readable by the parser that fills the bench line's roofline.traffic
(the field is null when a summary is stale, never because it cannot be
parsed)."""
import glob
import os

import bench


def test_counter_summaries_parse():
    paths = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "*_hbm_counters.md")))
    assert paths, "no committed counter summaries"
    for p in paths:
        sha, hbm = bench.parse_counter_summary(open(p).read())
        assert sha is not None and len(sha) == 64, p
        assert hbm is not None and hbm > 0, p


def test_counter_summary_parser_rejects_missing_fields():
    assert bench.parse_counter_summary("nothing here") == (None, None)
    sha = "ab" * 32
    text = f"source sha256 (over the four files, in that order): {sha}\nhbm_bytes_per_launch: 1.5e9\n"
    assert bench.parse_counter_summary(text) == (sha, 1.5e9)


def test_cpu_model_is_a_string_or_none():
    import bench
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
