"""The arrival protocols of the split merge, modelled on the CPU and checked
over every interleaving of the splits' steps (no GPU).

Each split of a query row ends its tile loop with a partial result that one
of them merges.  Two protocols are used by the forward kernel:

* last to arrive: every split stores its partial (the store is complete
  before the next step), then adds one to the row's counter; the split that
  sees nsplit - 1 merges every stored partial and sets the counter back to 0;
* two splits: each split first adds one to the counter's lower half; the
  first to arrive stores its partial and then adds one to the upper half;
  the second waits until the upper half is non-zero, sets the counter back
  to 0 and merges the stored partial with its own, which it never stores.

The model explores every order of the splits' atomic steps and checks that
the run always ends (no split waits forever), that exactly one split merges,
that it reads only partials already stored, and that the counter is 0 again
for the next call.  Planted mistakes (counting before storing, resetting the
counter before the wait) are caught.
"""

import pytest

LOW, HIGH = 1, 1 << 16


def _run_all(make_steps, n):
    """Every interleaving of the atomic steps of n splits.  make_steps(x,
    shared, k) takes split x's step k on the shared state and returns
    "step", "done" or "wait" (the step cannot be taken now).  Returns the
    final states: (shared state, per split None when finished, else the
    steps taken so far)."""
    finals = []

    def explore(shared, gens_state):
        progressed = False
        for x in range(n):
            hist = gens_state[x]
            if hist is None:
                continue                                  # finished
            sh = dict(shared, stored=set(shared["stored"]), merged=list(shared["merged"]),
                      bad=list(shared["bad"]))
            res = make_steps(x, sh, len(hist))
            if res == "wait":
                continue
            progressed = True
            new_state = list(gens_state)
            new_state[x] = None if res == "done" else hist + (1,)
            explore(sh, tuple(new_state))
        if not progressed:
            finals.append((shared, gens_state))

    explore({"counter": 0, "stored": set(), "merged": [], "bad": []}, tuple(() for _ in range(n)))
    return finals


def _last_to_arrive_step(n, count_before_store=False):
    """Step k of split x under the last-to-arrive protocol; mutates sh."""
    def step(x, sh, k):
        order = ["count", "store"] if count_before_store else ["store", "count"]
        if k < 2:
            op = order[k]
            if op == "store":
                sh["stored"].add(x)
            else:
                old = sh["counter"]
                sh["counter"] += LOW
                sh["last_" + str(x)] = old == n - 1
            return "step"
        if k == 2:
            if not sh.get("last_" + str(x)):
                return "done"
            sh["counter"] = 0
            sh["merged"].append(x)
            missing = set(range(n)) - sh["stored"]
            if missing:
                sh["bad"].append(("read before stored", x, sorted(missing)))
            return "done"
    return step


def _two_split_step(count_before_store=False, reset_early=False):
    """Step k of split x under the two-split protocol; mutates sh."""
    def step(x, sh, k):
        role = sh.get("role_" + str(x))
        if k == 0:
            old = sh["counter"]
            sh["counter"] += LOW
            sh["role_" + str(x)] = "first" if (old & 0xFFFF) == 0 else "second"
            return "step"
        if role == "first":
            order = ["count", "store"] if count_before_store else ["store", "count"]
            op = order[k - 1]
            if op == "store":
                sh["stored"].add(x)
            else:
                sh["counter"] += HIGH
            return "done" if k == 2 else "step"
        # second to arrive
        if k == 1:
            if reset_early:
                sh["counter"] = 0
                return "step"
            if sh["counter"] >> 16 == 0:
                return "wait"
            sh["counter"] = 0
            return "step"
        if k == 2:
            if reset_early and sh["counter"] >> 16 == 0 and (1 - x) not in sh["stored"]:
                return "wait"
            sh["merged"].append(x)
            if (1 - x) not in sh["stored"]:
                sh["bad"].append(("read before stored", x))
            if x in sh["stored"]:
                sh["bad"].append(("stored its own partial", x))
            return "done"
    return step


def _check(finals, n):
    problems = []
    for sh, st in finals:
        if any(h is not None for h in st):
            problems.append("a split waits forever")
        if len(sh["merged"]) != 1:
            problems.append("merged %d times" % len(sh["merged"]))
        problems += [str(b) for b in sh["bad"]]
        if sh["counter"] != 0:
            problems.append("counter left at %#x" % sh["counter"])
    return sorted(set(problems))


@pytest.mark.parametrize("n", [2, 3, 4])
def test_last_to_arrive_protocol(n):
    finals = _run_all(_last_to_arrive_step(n), n)
    assert finals
    assert _check(finals, n) == []


def test_last_to_arrive_catches_counting_before_storing():
    finals = _run_all(_last_to_arrive_step(3, count_before_store=True), 3)
    assert any("read before stored" in p for p in _check(finals, 3))


def test_two_split_protocol():
    finals = _run_all(_two_split_step(), 2)
    assert len(finals) > 2                          # several orders explored
    assert _check(finals, 2) == []


def test_two_split_catches_counting_stored_before_storing():
    finals = _run_all(_two_split_step(count_before_store=True), 2)
    assert any("read before stored" in p for p in _check(finals, 2))


def test_two_split_catches_resetting_before_the_wait():
    finals = _run_all(_two_split_step(reset_early=True), 2)
    assert any("counter left" in p for p in _check(finals, 2))
