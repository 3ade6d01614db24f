"""Helpers shared by the GPU tests: comparisons and oracle-side reference runs."""
import numpy as np
import pytest

try:  # import early: the first import on a fresh machine is slow
    import torch  # noqa: F401
except ImportError:  # pragma: no cover
    torch = None

import oracle


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_verify_amd as tv
    tv.lib()  # raises if the library is missing: no silent fallback
    return torch


GUARD_BYTES = 4096
GUARD_BYTE = 0xA5


class Guarded:
    """A device output buffer inside a larger allocation whose GUARD_BYTES
    before and after hold a sentinel byte: check() fails when a kernel wrote
    outside the buffer it was given.  The buffer itself starts 4096 bytes in,
    so it keeps the allocation's alignment."""

    def __init__(self, torch, shape, dtype, device="cuda"):
        n = 1
        for k in shape:
            n *= int(k)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((2 * GUARD_BYTES + nbytes,), GUARD_BYTE, dtype=torch.uint8, device=device)
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(*shape)
        self.t.zero_()

    def check(self, what="buffer"):
        lo = self.raw[:GUARD_BYTES].cpu().numpy()
        hi = self.raw[-GUARD_BYTES:].cpu().numpy()
        bad_lo = int(np.count_nonzero(lo != GUARD_BYTE))
        bad_hi = int(np.count_nonzero(hi != GUARD_BYTE))
        assert bad_lo == 0 and bad_hi == 0, "%s: %d bytes before and %d after it were overwritten" % (
            what, bad_lo, bad_hi)


def guarded_runner_class():
    """VerifyRunner whose every buffer (workspace, residual, tree K/V, logits,
    argmax, gap, path, committed) sits inside guard bands; check_guards()
    asserts none was touched."""
    import torch
    from tree_verify_amd.runner import VerifyRunner

    class GuardedRunner(VerifyRunner):
        def _zeros(self, shape, dtype):
            g = Guarded(torch, shape, dtype, self.device)
            self.__dict__.setdefault("_guards", []).append(g)
            return g.t

        def check_guards(self):
            torch.cuda.synchronize()
            for i, g in enumerate(self._guards):
                g.check("runner buffer %d" % i)

    return GuardedRunner


def bf16_bits_to_f64(t):
    """Device/host int16 tensor of bf16 bits -> fp64 numpy."""
    a = t.detach().cpu().numpy().view(np.uint16)
    return oracle.bf16_to_f64(a)


def row_rel_err(got, ref):
    """Per-row max |got - ref| / max |ref| (the inf-norm relative error)."""
    got = np.asarray(got, np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    return np.max(np.abs(got - ref), axis=1) / np.maximum(np.max(np.abs(ref), axis=1), 1e-30)


def decisive_compare(parent, tokens, oracle_am, oracle_gap, gpu_am, gpu_path, gpu_len,
                     gpu_committed, thr=0.05):
    """Greedy tokens must match wherever the oracle's top1-top2 gap exceeds thr;
    the path must match exactly when every oracle-accepted node is decisive.
    On every run, decided or not, the GPU's walk must be exactly the oracle's
    walk over the GPU's own greedy tokens (bit-exact path, length and
    committed tokens).  Returns (n_decisive_tokens, path_decided)."""
    dec = oracle_gap > thr
    bad = [i for i in range(len(oracle_am)) if dec[i] and gpu_am[i] != oracle_am[i]]
    assert not bad, "greedy token mismatch at decisive nodes %s" % bad
    wpath, wcommitted = oracle.accept_path(parent, tokens, [int(a) for a in gpu_am])
    assert int(gpu_len) == len(wpath), "walk length %d, oracle walk over the GPU tokens %d" % (gpu_len, len(wpath))
    assert list(gpu_path[:gpu_len]) == list(wpath), "walk differs from the oracle walk over the GPU tokens"
    assert list(gpu_committed[:gpu_len]) == list(wcommitted), "committed tokens differ"
    path, committed = oracle.accept_path(parent, tokens, oracle_am)
    # nodes whose greedy token the acceptance actually consulted
    acc_nodes = _accepted_nodes(parent, tokens, oracle_am)
    decided = all(dec[i] for i in acc_nodes)
    if decided:
        assert list(gpu_path[:gpu_len]) == list(path)
        assert list(gpu_committed[:gpu_len]) == list(committed)
    return int(dec.sum()), decided


def _accepted_nodes(parent, tokens, am):
    acc = [True] + [False] * (len(parent) - 1)
    for i in range(1, len(parent)):
        acc[i] = acc[parent[i]] and int(tokens[i]) == int(am[parent[i]])
    return [i for i in range(len(parent)) if acc[i]]
