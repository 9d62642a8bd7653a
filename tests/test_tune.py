"""The tile/occupancy sweep's bookkeeping (CPU): the header it writes from a
sweep's printed lines names the fastest setting of each group, keeps the
current values of a group that was not swept, and the committed header
defines every knob the sweep knows."""
import json

from attention_pass_cascaded_amd import tune


def test_committed_header_defines_every_knob():
    for group in tune.GROUPS.values():
        for knob in group["knobs"]:
            assert tune.current_value(knob) in group["knobs"][knob]


def test_header_from_log_picks_the_fastest(tmp_path):
    hdr = tmp_path / "tuned.hpp"
    hdr.write_text(open(tune.HEADER).read())
    log = tmp_path / "sweep.log"
    rows = [{"group": "fwd", "setting": {"RF_FWD_WAVES_D64": w}, "ms": {"prefill:x:causal": t}, "total_ms": t}
            for w, t in ((2, 0.20), (3, 0.15), (4, 0.17))]
    log.write_text("noise\n" + "\n".join(json.dumps(r) for r in rows) + "\n")
    winners = tune.header_from_log(str(log), str(hdr))
    assert winners["fwd"] == {"RF_FWD_WAVES_D64": 3}
    assert tune.current_value("RF_FWD_WAVES_D64", str(hdr)) == 3
    for knob in tune.GROUPS["bwd"]["knobs"]:           # not swept: unchanged
        assert tune.current_value(knob, str(hdr)) == tune.current_value(knob)
    text = hdr.read_text()
    assert "RF_FWD_WAVES_D64=2: prefill causal 0.2000" in text and "#pragma once" in text
