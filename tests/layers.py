"""The full-size synthetic layers, generated once per test session.

synth.make_layer is deterministic in the configuration name; the largest layer takes
tens of seconds to draw and split, so the GPU tests that sample it share one copy."""
import functools

import synth


@functools.lru_cache(maxsize=2)
def layer(name):
    return synth.make_layer(name)
