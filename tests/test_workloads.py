"""The workload file (synth/workloads.json) is the one place the five workloads
are defined: synth.SHAPES is read from it, and its generator parameters are the
generators' own defaults (CPU only)."""
import inspect
import json

import synth


def test_shapes_come_from_the_workload_file():
    doc = json.load(open(synth.WORKLOADS_JSON))
    names = [w["name"] for w in doc["workloads"]]
    assert list(synth.SHAPES) == names
    for w in doc["workloads"]:
        s = synth.SHAPES[w["name"]]
        assert (s.hidden, s.experts, s.top_k, s.inter, s.layers, s.tokens, s.shared, s.steps) == \
            (w["hidden"], w["experts"], w["top_k"], w["inter"], w["layers"], w["tokens"],
             w["shared"], w["steps"])
        assert s.fmt == synth.FMT_NAMES[w["format"]]
    # the cache sizes the measurements quote
    assert synth.SHAPES["decode_bf16_48L"].cache_slots == 2273  # 37% of 48 x 128
    assert synth.SHAPES["decode_mxfp4_43L"].cache_slots == 1210  # 11% of 43 x 256
    assert synth.SHAPES["prefill_decode_nvfp4_8L"].cache_slots == 512  # two layers' experts


def test_generator_parameters_are_the_generators_defaults():
    g = json.load(open(synth.WORKLOADS_JSON))["generators"]
    trace = inspect.signature(synth.sticky_zipf_trace).parameters
    assert trace["alpha"].default == g["trace_zipf_alpha"]
    assert trace["p_keep"].default == g["trace_keep_probability"]
    assert inspect.signature(synth.router_weights).parameters["sigma"].default == g["router_sigma"]
    assert inspect.signature(synth.expert_block).parameters["sigma"].default == g["weight_sigma"]
