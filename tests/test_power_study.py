"""The power study's reading of the system management tool's output (host
only): one query's socket power and the mean of the graphics clock domains,
from a captured `amd-smi metric -p -c -g 0` listing of an idle MI355X (below,
as the tool printed it), and no sample when the tool is missing or prints
nothing usable."""
import subprocess
import types

from block_sparse_cross_amd import power_study

LISTING = """\
GPU: 0
    POWER:
        SOCKET_POWER: 247 W
        GFX_VOLTAGE: N/A
        SOC_VOLTAGE: N/A
        MEM_VOLTAGE: N/A
        THROTTLE_STATUS: N/A
        POWER_MANAGEMENT: N/A
    CLOCK:
        GFX_0:
            CLK: 94 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        GFX_1:
            CLK: 95 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        GFX_2:
            CLK: 94 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        GFX_3:
            CLK: 94 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        GFX_4:
            CLK: 95 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        GFX_5:
            CLK: 95 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        GFX_6:
            CLK: 114 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        GFX_7:
            CLK: 115 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
            DEEP_SLEEP: ENABLED
        MEM_0:
            CLK: 2000 MHz
            MIN_CLK: 2000 MHz
            MAX_CLK: 2000 MHz
            DEEP_SLEEP: DISABLED
        VCLK_0:
            CLK: 59 MHz
        VCLK_1:
            CLK: 59 MHz
        VCLK_2:
            CLK: 59 MHz
        VCLK_3:
            CLK: 59 MHz
        DCLK_0:
            CLK: 48 MHz
        DCLK_1:
            CLK: 48 MHz
        DCLK_2:
            CLK: 48 MHz
        DCLK_3:
            CLK: 48 MHz
        SOCCLK_0:
            CLK: 38 MHz
"""


def fake_run(text):
    def run(cmd, **kw):
        assert cmd[0] == power_study.SMI and cmd[1] == "metric"
        return types.SimpleNamespace(stdout=text, returncode=0)
    return run


def test_sample_from_captured_listing(monkeypatch):
    monkeypatch.setattr(subprocess, "run", fake_run(LISTING))
    power, clock = power_study.sample_once()
    assert power == 247
    # eight graphics clock domains (94, 95, 94, 94, 95, 95, 114, 115 MHz); memory, video
    # and SoC clocks are not counted
    assert abs(clock - (94 + 95 + 94 + 94 + 95 + 95 + 114 + 115) / 8) < 1e-9


def test_no_sample_without_the_tool(monkeypatch):
    def missing(cmd, **kw):
        raise FileNotFoundError(cmd[0])
    monkeypatch.setattr(subprocess, "run", missing)
    assert power_study.sample_once() is None
    monkeypatch.setattr(subprocess, "run", fake_run("no devices\n"))
    assert power_study.sample_once() is None
