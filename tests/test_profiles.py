"""The figures written into profiles/ agree with their own arithmetic.

Every sentence of the form "<bytes> MB ... / <t> us = <rate> TB/s, <p>% of
the 8 TB/s peak" must have rate = bytes / t and p = rate / 8 TB/s (to the
printed digits), and every traffic record's total must equal its read plus
write bytes, each the raw counter scaled by the calibration factor it states.
"""
import glob
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RATE = re.compile(r"([\d.]+) MB[^=]*?/ ([\d.]+) us = ([\d.]+) TB/s, ([\d.]+)% of the 8 TB/s peak")
FLOPS = re.compile(r"([\d.]+) GFLOP[^=]*?/ ([\d.]+) us = ([\d.]+) TFLOP/s, ([\d.]+)% of the ([\d.]+) TFLOP/s peak")


def _md():
    return sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


def test_rate_sentences_add_up():
    seen = 0
    for path in _md():
        text = " ".join(open(path).read().split())
        for mb, us, tbs, pct in RATE.findall(text):
            rate = float(mb) * 1e6 / (float(us) * 1e-6) / 1e12
            assert abs(rate - float(tbs)) <= 0.006 + 1e-3 * rate, (path, mb, us, tbs)
            assert abs(rate / 8.0 * 100 - float(pct)) <= 0.06 + 1e-3 * rate * 12.5, (path, tbs, pct)
            seen += 1
        for gf, us, tf, pct, peak in FLOPS.findall(text):
            rate = float(gf) * 1e9 / (float(us) * 1e-6) / 1e12
            assert abs(rate - float(tf)) <= 0.6 + 1e-3 * rate, (path, gf, us, tf)
            assert abs(rate / float(peak) * 100 - float(pct)) <= 0.06 + 1e-3 * rate / float(peak) * 100, (path, pct)
            seen += 1
    assert seen >= 1


def test_traffic_records_add_up():
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")):
        d = json.load(open(path))
        assert d["hbm_bytes_per_launch"] == d["hbm_read_bytes_per_launch"] + d["hbm_write_bytes_per_launch"], path
        assert 1.9 < d["fetch_scale"] < 2.1 and 0.9 < d["write_scale"] < 1.1, path
        if "fetch_kib_raw_mean" in d:
            assert abs(d["fetch_kib_raw_mean"] * 1024 * d["fetch_scale"] - d["hbm_read_bytes_per_launch"]) \
                <= 1e-6 * d["hbm_read_bytes_per_launch"] + 1024, path
            assert abs(d["write_kib_raw_mean"] * 1024 * d["write_scale"] - d["hbm_write_bytes_per_launch"]) \
                <= 1e-6 * d["hbm_write_bytes_per_launch"] + 1024, path
