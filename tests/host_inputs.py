"""Host copies of the synthetic workloads' tensors (from ``synth``), for the
oracle side of the tests."""
import numpy as np

import synth
from synth.workloads import weight_spec


class HostWeights:
    """``w(name)`` -> uint16 array of a stored weight, generated on first use.
    With ``keep_blocks`` the arrays of at most that many blocks stay cached, so
    a large model can be walked one block at a time."""

    def __init__(self, g, keep_blocks=None):
        self.g = g
        self.spec = {name: (tid, shape, mean, std) for name, tid, shape, mean, std in weight_spec(g)}
        self.cache = {}
        self.keep_blocks = keep_blocks
        self.order = []

    def __call__(self, name):
        if name not in self.cache:
            tid, shape, mean, std = self.spec[name]
            arr = synth.normal_bf16(int(np.prod(shape)), self.g.weight_seed, tid, mean, std)
            self.cache[name] = arr.reshape(shape)
            if self.keep_blocks is not None and name.startswith("b"):
                blk = name.split(".")[0]
                if blk not in self.order:
                    self.order.append(blk)
                while len(self.order) > self.keep_blocks:
                    old = self.order.pop(0)
                    for k in [k for k in self.cache if k.startswith(old + ".")]:
                        del self.cache[k]
        return self.cache[name]

    def all(self):
        return {name: self(name) for name in self.spec}


def prompt(g, seq=0, n=None):
    n = g.prompt_len if n is None else n
    return synth.tokens(n, g.prompt_seeds[seq], 0, g.vocab)
