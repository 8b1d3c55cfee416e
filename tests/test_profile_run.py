"""Host logic of the profiling launcher: the amd-smi reading parser."""
import json

import pytest

pytest.importorskip("torch")

from exact_attention_48_amd.profile_run import parse_smi_metrics  # noqa: E402


def _doc(power, clocks):
    clock = {f"gfx_{i}": {"clk": {"value": c, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                          "max_clk": {"value": 2400, "unit": "MHz"}} for i, c in enumerate(clocks)}
    clock["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    return json.dumps({"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": power, "unit": "W"},
                                                         "gfx_voltage": "N/A"}, "clock": clock}]})


def test_power_and_mean_gfx_clock():
    pw, ck = parse_smi_metrics(_doc(1353, [1700, 1800, 1750, 1750, 1700, 1800, 1750, 1750]))
    assert pw == 1353.0 and ck == 1750.0          # memory and min/max clocks are not gfx clocks


def test_missing_readings_are_none():
    pw, ck = parse_smi_metrics(json.dumps({"gpu_data": [{"gpu": 0, "power": {"socket_power": "N/A"}}]}))
    assert pw is None and ck is None
    with pytest.raises(ValueError):
        parse_smi_metrics("not json")
