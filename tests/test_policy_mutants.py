"""Mutation tests of the serving-policy oracle's pins: each mutant breaks one
of the simulation's stated rules (a text replacement in the oracle's source,
executed as a module of its own) and must fail at least one of the oracle's
own pins in test_policy_sim (closed forms, SplitMix64's published outputs,
the memory-cap scenario); the native simulator is not used as a pin here."""

import inspect
import types

import pytest

import test_policy_sim as tp
from oracle import policy_oracle as po

SRC = inspect.getsource(po)

MUTANTS = {
    # rule 1: admission needs the prompt's blocks plus one spare
    "admission-without-spare": ('if free < need + 1:', 'if free < need:'),
    # rule 2: a new block when the length is a multiple of the block size
    "block-boundary-off-by-one": ('if s["len"] % bs == 0:', 'if s["len"] % bs == 1:'),
    # rule 2: preemption takes the most recently admitted sequence
    "preempts-oldest": ('victim = running.pop()', 'victim = running.pop(0)'),
    # rule 2: a preempted request goes back to the front of the queue
    "preempted-to-back": ('waiting.insert(0, victim["req"])', 'waiting.append(victim["req"])'),
    # rule 3: finished sequences free their blocks
    "finished-keep-blocks": ('        for s in [s for s in running if s["left"] <= 0]:\n            free += s["blocks"]\n',
                             ''),
    # rule 4: eligibility is length - watermark >= W
    "strict-eligibility": ('if s["len"] - s["wm"] < W:', 'if s["len"] - s["wm"] <= W:'),
    # rule 4: the watermark moves to the new length minus B
    "watermark-at-new-length": ('s["wm"] = s["len"] - B', 's["wm"] = s["len"]'),
    # rule 4: new length L - (W - B) + R
    "length-drops-protected": ('s["len"] = s["len"] - (W - B) + R', 's["len"] = s["len"] - W + R'),
    # rule 4: threshold compression costs per cached key
    "threshold-cost-per-sequence": ('c_ms += cfg["compress_ms_per_key"] * s["len"]',
                                    'c_ms += cfg["compress_ms_per_key"]'),
    # rule 5: decode time counts the tokens cached when the step starts
    "decode-time-after-append": (
        '        ms = cfg["decode_ms_fixed"] + cfg["decode_ms_per_token"] * sum(s["len"] for s in running)\n',
        '        ms = cfg["decode_ms_fixed"] + cfg["decode_ms_per_token"] * sum(s["len"] + 1 for s in running)\n'),
    # request lengths: gen_min + x % (gen_max - gen_min + 1)
    "length-range-short": ('% (cfg["gen_max"] - cfg["gen_min"] + 1)', '% (cfg["gen_max"] - cfg["gen_min"])'),
    # SplitMix64: the state is advanced by the golden gamma before mixing
    "splitmix-no-increment": ('z = (x + 0x9E3779B97F4A7C15) & MASK', 'z = x & MASK'),
}


def _oracle_pins():
    tp.test_splitmix64_published_outputs()
    tp.test_rule_request_lengths_cover_the_range()       # before any pin with gen_min == gen_max
    for name in sorted(dir(tp)):
        if name.startswith("test_rule_"):
            getattr(tp, name)()
    tp.test_one_request_without_compression()
    for gen in (28, 29, 113, 114, 500):
        tp.test_periodic_one_sequence_closed_form(gen)
    for gen in (30, 31, 90, 200):
        tp.test_threshold_one_sequence_closed_form(gen)
    tp.test_sequential_service_with_one_slot()
    tp.test_memory_cap_stalls_and_preemption()


def _mutated(kind):
    old, new = MUTANTS[kind]
    assert SRC.count(old) == 1, kind
    mod = types.ModuleType("policy_oracle_mutant")
    exec(compile(SRC.replace(old, new), "policy_oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_pins_pass_on_the_oracle():
    _oracle_pins()


@pytest.mark.parametrize("kind", list(MUTANTS))
def test_pins_reject_mutant(kind, monkeypatch):
    mod = _mutated(kind)
    for name in ("splitmix64", "gen_length", "simulate"):
        monkeypatch.setattr(po, name, getattr(mod, name))
    with pytest.raises(AssertionError):
        _oracle_pins()
