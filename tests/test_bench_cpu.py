"""CPU tests of bench.py's kernel timing arithmetic (no GPU): with stop
events only, a call's time runs from the previous call's end to its own, so
the calls of the timed region add up to its length; a call with a start
event (the Lloyd fit) is timed from that start; arm() hands the right
events to the library; the oracle baseline's passes repeat until their time
is spent."""
import bench


class FakeEvent:
    """A recorded timestamp in milliseconds."""

    def __init__(self, t):
        self.t = t

    def elapsed_time(self, end):
        return end.t - self.t


def timer(names, stamps, spans=(), starts=None):
    """A bench.Timer whose events carry the given timestamps: stamps[i][n]
    is the end of call n in step i, starts[i][n] its start (spans only)."""
    tm = object.__new__(bench.Timer)
    tm.names = list(names)
    tm.spans = set(spans)
    tm.start = FakeEvent(0.0)
    tm.ev = [{n: (FakeEvent(starts[i][n]) if n in tm.spans else None, FakeEvent(stamps[i][n])) for n in names}
             for i in range(len(stamps))]
    tm.end = FakeEvent(stamps[-1][names[-1]] + 0.001)
    return tm


def test_stop_only_intervals_chain_and_add_up():
    # two calls per step: encode ends at 0.036, decode at 0.064, ...
    stamps = [{"encode": 0.036, "decode": 0.064}, {"encode": 0.101, "decode": 0.129},
              {"encode": 0.166, "decode": 0.193}]
    tm = timer(["encode", "decode"], stamps)
    enc, dec = tm.per_kernel_ms("encode"), tm.per_kernel_ms("decode")
    assert [round(x, 6) for x in enc] == [0.036, 0.037, 0.037]
    assert [round(x, 6) for x in dec] == [0.028, 0.028, 0.027]
    assert abs(sum(enc) + sum(dec) - stamps[-1]["decode"]) < 1e-12


def test_span_call_timed_from_its_start():
    stamps = [{"fit": 1.6}, {"fit": 3.2}]
    starts = [{"fit": 0.1}, {"fit": 1.7}]
    tm = timer(["fit"], stamps, spans=("fit",), starts=starts)
    assert [round(x, 6) for x in tm.per_kernel_ms("fit")] == [1.5, 1.5]


def test_arm_passes_the_step_events():
    calls = []

    class FakeTQ:
        @staticmethod
        def time_next_call(start, stop):
            calls.append((start, stop))

    ev = {"encode": (None, "stop-e"), "fit": ("start-f", "stop-f")}
    bench.arm(FakeTQ, ev, "encode")
    bench.arm(FakeTQ, ev, "fit")
    bench.arm(FakeTQ, None, "encode")  # outside the timed region: nothing
    assert calls == [(None, "stop-e"), ("start-f", "stop-f")]


def test_passes_run_until_the_time_is_spent():
    t = iter([0.3, 0.3, 0.3, 0.3, 0.3])
    assert bench._passes(lambda: next(t), min_s=1.0) == (0.3, 4)
    assert bench._passes(lambda: 2.0, min_s=1.0) == (2.0, 1)
    assert bench._passes(lambda: 0.01, min_s=1.0, max_passes=16) == (0.01, 16)
