"""Host-side helpers of bench.py (no GPU): the shader-clock reading."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_read_sclk_takes_the_marked_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1712Mhz *\n2: 2400Mhz\n")
    assert bench.read_sclk(str(f)) == 1712.0


def test_read_sclk_without_a_mark_or_file(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk(str(f)) is None
    assert bench.read_sclk(str(tmp_path / "missing")) is None
