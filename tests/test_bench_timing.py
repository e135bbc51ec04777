"""The bench's trial timer (bench.Timed), on the CPU with a stand-in for
torch.cuda: a trial whose spin hold ended before its launches were all
enqueued (the start event already passed) is run again with twice the hold,
at most `retries` times, and the kept time is the last attempt's."""
import types

import pytest

import bench


class _Cuda:
    def __init__(self, passed, times):
        self.passed = list(passed)  # what each start event's query() returns, in order
        self.times = list(times)    # ms between the events of each kept attempt, in order
        self.holds = []

    def synchronize(self):
        pass

    def current_stream(self):
        return None

    def _sleep(self, cycles):
        self.holds.append(cycles)

    def Event(self, enable_timing=False):
        cuda = self

        class Ev:
            def record(self, stream=None):
                pass

            def query(self):
                return cuda.passed.pop(0)

            def elapsed_time(self, other):
                return cuda.times.pop(0)

        return Ev()


@pytest.fixture
def fake_torch(monkeypatch):
    monkeypatch.setattr(bench.Timed, "cycles_per_ms", 1000.0)
    monkeypatch.setattr(bench.Timed, "redone", 0)

    def make(passed, times):
        cuda = _Cuda(passed, times)
        return types.SimpleNamespace(cuda=cuda), cuda
    return make


def test_clean_trials_are_kept_as_they_are(fake_torch):
    torch, cuda = fake_torch([False, False, False], [1.0, 2.0, 3.0])
    calls = []
    t = bench.Timed(torch, calls.append, steps=10, warmup=2, trials=3)
    assert bench.Timed.redone == 0
    assert t.us == [100.0, 200.0, 300.0] and t.median == 200.0  # ms / steps, in us
    assert cuda.holds == [1000.0 * (2.0 + 10 * 0.04)] * 3
    assert len(calls) == 2 + 3 * 10


def test_a_drained_trial_is_run_again_with_twice_the_hold(fake_torch):
    # trial 0: drained once, then clean; trial 1: clean (a drained attempt's
    # events are never read)
    torch, cuda = fake_torch([True, False, False], [1.0, 1.5])
    calls = []
    t = bench.Timed(torch, calls.append, steps=10, warmup=0, trials=2)
    assert bench.Timed.redone == 1
    assert t.us == [100.0, 150.0]
    h = 1000.0 * (2.0 + 10 * 0.04)
    assert cuda.holds == [h, 2 * h, 2 * h]  # the longer hold stays for later trials
    assert len(calls) == 3 * 10


def test_retries_are_bounded(fake_torch):
    torch, cuda = fake_torch([True] * 3, [7.0])
    t = bench.Timed(torch, lambda i: None, steps=4, warmup=0, trials=1, retries=2)
    assert bench.Timed.redone == 2
    assert t.us == [7.0 * 1e3 / 4]  # the last attempt is kept
    assert len(cuda.holds) == 3


def test_the_hold_is_capped_across_trials(fake_torch):
    # a trial that never passes the check (the host blocks until the GPU
    # has drained) must not make later holds grow without bound
    torch, cuda = fake_torch([True] * 6, [1.0, 1.0])
    bench.Timed(torch, lambda i: None, steps=4, warmup=0, trials=2, retries=2)
    h = 1000.0 * (2.0 + 4 * 0.04)
    assert cuda.holds == [h, 2 * h, 4 * h, 4 * h, 4 * h, 4 * h]


def test_no_retries_keeps_every_first_attempt(fake_torch):
    torch, cuda = fake_torch([True, True], [1.0, 2.0])
    t = bench.Timed(torch, lambda i: None, steps=5, warmup=0, trials=2, retries=0)
    assert bench.Timed.redone == 0 and t.us == [200.0, 400.0] and len(cuda.holds) == 2
