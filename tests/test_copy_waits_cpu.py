"""Copy waits of the kernels that count their own copies, checked on the host
against their issue order: the producer/consumer tiles, the register-operand
forward, the ping-pong tiles and the line-staged small-M forward.

The producer waves of the (BM x BN) tiled kernel issue LDS-direct copies that
complete in issue order and wait on them with vmcnt(c), i.e. until at most c of
their own copies are still in flight.  This test replays the issue order (the
prologue's activation and weight copies, then per step the activation copy of
step i+NA-1 and the weight copy of step i+PD) and checks that every wait the
kernel takes guarantees the copies the next step reads: all prologue copies
before the first expansion, the weights of step 1 before step 0, and at the
end of step i the activation tile of step i+1 and the packed weights of step
i+2.  The wait expressions are read from the kernel source, so an edit to them
is checked here.
"""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "nf4_bit_weight_amd", "csrc", "nf4_gemm.hip")


def _expr(text, pattern):
    m = re.search(pattern, text, re.S)
    assert m, pattern
    e = m.group(1)
    # the only conditional form used: (a > b ? c : d)
    e = re.sub(r"\(([^()?]+)\?([^():]+):([^()]+)\)", r"((\2) if (\1) else (\3))", e)
    return e


def _wait_exprs():
    s = open(SRC).read()
    return {
        "after_a": _expr(s, r"constexpr int kAfterA = ([^;]+);"),
        "after_w": _expr(s, r"constexpr int kAfterW = ([^;]+);"),
        "pro1": _expr(s, r"wait_vm\(ic<(\(PD - 1\) \* kW)>\{\}\);"),
        "pro2": _expr(s, r"expand_into\(0, 0, 0\);.*?wait_vm\(ic<(.+?)>\{\}\);"),
    } if "expand_into(0, 0, 0);" in s else None


def _replay(NA, PD, kA, kW, n, ex):
    env = {"NA": NA, "PD": PD, "kA": kA, "kW": kW}
    k_wait = min(eval(ex["after_a"], {"__builtins__": {}}, env), eval(ex["after_w"], {"__builtins__": {}}, env))
    ops = []
    done = 0                                   # ops[:done] known complete

    def issue(kind, step, count):
        ops.extend([(kind, step)] * count)

    def wait(c):
        nonlocal done
        done = max(done, len(ops) - c)

    def landed(kind, step):
        return max(k for k, o in enumerate(ops) if o == (kind, step)) < done

    for j in range(NA - 1):
        issue("A", j, kA)
    for j in range(PD):
        issue("W", j, kW)
    wait(eval(ex["pro1"], {"__builtins__": {}}, env))
    assert all(landed("A", j) for j in range(NA - 1)) and landed("W", 0), "prologue"
    wait(eval(ex["pro2"], {"__builtins__": {}}, env))
    if n > 1:
        assert landed("W", 1), "weights of step 1 before step 0"
    for i in range(n):
        issue("A", i + NA - 1, kA)
        issue("W", i + PD, kW)
        wait(k_wait)
        if i + 1 < n:
            assert landed("A", i + 1), f"end of step {i}: activation tile of step {i + 1}"
        if i + 2 < n:
            assert landed("W", i + 2), f"end of step {i}: weights of step {i + 2}"


@pytest.mark.parametrize("NA,PD", [(4, 4), (2, 4), (2, 2)])
def test_copy_waits_cover_every_read(NA, PD):
    ex = _wait_exprs()
    assert ex is not None, "prologue not found in the kernel source"
    for kA in (1, 2, 4, 8, 16):               # activation copy instructions per wave
        for kW in (3, 4):                     # weight copy instructions (plain, nested)
            for n in range(1, 14):
                _replay(NA, PD, kA, kW, n, ex)


def test_replay_catches_the_steady_state_wait_in_the_prologue():
    """The first step of four-deep rings needs the prologue's stricter wait:
    with the weights of step 1 as the prologue's only requirement, the end of
    step 0 leaves part of the weight copy of step 2 in flight."""
    ex = dict(_wait_exprs())
    ex["pro2"] = "(PD - 2) * kW"
    with pytest.raises(AssertionError, match="weights of step 2"):
        _replay(4, 4, 2, 3, 4, ex)


# ---- the register-operand forward kernel -------------------------------------------
# Its producer work is done by every wave: a prologue W0 A0 W1 A1 W2 (only the
# steps that exist), then during step i the activation copy of step i+2 (in
# slices 0-2) and the weight copy of step i+3 (in slice 3), again only for
# steps that exist.  Step i first waits for the weights of step i+1 (it
# expands them during its slices) and ends with its part of A(i+1) landed.
# Each wait is a chain of cases by how many of the later copies exist; the
# chains are read from the kernel source.

def _chain(text, pattern):
    m = re.search(pattern, text, re.S)
    assert m, pattern
    return m.group(1)


def _cases(chain):
    """`if (c1) wait_vm(ic<e1>{}); else if (c2) wait_vm(ic<e2>{}); else wait_vm(ic<e3>{});`
    as [(condition or None, expression)]."""
    out = []
    for cond, expr in re.findall(r"(?:else\s+)?(?:if\s*\(([^)]*)\)\s*)?wait_vm\(ic<([^>]+)>\{\}\);", chain):
        out.append((cond or None, expr))
    assert out, chain
    return out


def _rb_exprs():
    s = open(SRC).read()
    body = s[s.index("void k_rb("):s.index("// Fixed-order sum of split partials")]
    ex = {
        "kcopies": _expr(body, r"constexpr int kCopies = ([^;]+);"),
        "pro_w0": _cases(_chain(body, r"// weights of step 0 landed[^\n]*\n(.*?wait_vm\(ic<kAJ>\{\}\);)")),
        "pro_a0": _cases(_chain(body, r"// own part of A\(0\) landed[^\n]*\n(.*?else wait_vm\(ic<0>\{\}\);)")),
        "step_w": _cases(_chain(body, r"// weights of step i\+1 landed[^\n]*\n(.*?else if \(i \+ 1 < n\) wait_vm\(ic<[^>]+>\{\}\);)").replace("FULL || ", "")),
        "step_a": _cases(_chain(body, r"// own part of A\(i\+1\) landed[^\n]*\n[^\n]*\n(.*?else wait_vm\(ic<0>\{\}\);)").replace("FULL || ", "")),
    }
    # the copies of a step go out only for steps that exist
    assert "if (kk < 3 && (FULL || i + 2 < n))" in body and "if (kk == 3 && (FULL || i + 3 < n)) issue_w(i + 3, P);" in body
    # a FULL step (three more steps after it) takes the first case of each chain
    assert "for (; i + 6 <= n; i += 3) {" in body
    assert "if (n > 1) {\n      issue_w(1, 1);\n      issue_a(1, 1);\n    }\n    if (n > 2) issue_w(2, 2);" in body
    return ex


def _replay_rb(kAJ, kWCopies, n, ex):
    env = {"kAJ": kAJ, "kWCopies": kWCopies, "n": n}
    env["kCopies"] = eval(ex["kcopies"], {"__builtins__": {}}, env)
    ops, done, issued = [], 0, set()

    def issue(kind, step, count):
        assert step < n, f"copy of step {step} past the end"
        assert (kind, step) not in issued, f"{kind}({step}) copied twice"
        issued.add((kind, step))
        ops.extend([(kind, step)] * count)

    def wait(key, **kw):
        nonlocal done
        for cond, expr in ex[key]:
            if cond is None or eval(cond, {"__builtins__": {}}, {**env, **kw}):
                done = max(done, len(ops) - eval(expr, {"__builtins__": {}}, env))
                return

    def landed(kind, step):
        return max(k for k, o in enumerate(ops) if o == (kind, step)) < done

    issue("W", 0, kWCopies)
    issue("A", 0, kAJ)
    if n > 1:
        issue("W", 1, kWCopies)
        issue("A", 1, kAJ)
    if n > 2:
        issue("W", 2, kWCopies)
    wait("pro_w0")
    assert landed("W", 0), "prologue: weights of step 0"
    wait("pro_a0")
    assert landed("A", 0), "prologue: activation tile of step 0"
    for i in range(n):
        wait("step_w", i=i)
        if i + 1 < n:
            assert landed("W", i + 1), f"step {i}: weights of step {i + 1}"
        if i + 2 < n:
            issue("A", i + 2, kAJ)
        if i + 3 < n:
            issue("W", i + 3, kWCopies)
        wait("step_a", i=i)
        if i + 1 < n:
            assert landed("A", i + 1), f"end of step {i}: activation tile of step {i + 1}"
    assert issued == {(k, j) for k in "AW" for j in range(n)}


def test_register_operand_copy_waits_cover_every_read():
    ex = _rb_exprs()
    for kAJ in (1, 2, 4, 8):
        for kWCopies in (2, 3):
            for n in range(1, 12):
                _replay_rb(kAJ, kWCopies, n, ex)


def test_register_operand_replay_catches_a_short_wait():
    ex = dict(_rb_exprs())
    ex["step_a"] = [("i + 3 < n", "kCopies + kWCopies + 1")] + ex["step_a"][1:]
    with pytest.raises(AssertionError, match="activation tile"):
        _replay_rb(2, 3, 6, ex)
    ex = dict(_rb_exprs())
    ex["step_w"] = [("i + 2 < n", "kCopies + 1")] + ex["step_w"][1:]
    with pytest.raises(AssertionError, match="weights of step"):
        _replay_rb(2, 3, 6, ex)


# ---- the ping-pong kernel ----------------------------------------------------------
# Per wave: a prologue A(0) (four copy groups), W(0), W(1), W(2) (kWc copies
# each: the packed bytes, plus a scale on waves 0-3 or a nested scale on
# waves 4-7 of the nested form), then a wait that leaves only W(2) in flight.
# Step i issues A(i + 1) (if there is a step i + 1) and then W(i + 3) (if
# there is a step i + 3) and ends with a wait that leaves only the newest
# weight copies in flight.  Step i reads A(i) and the weights of step i + 1.

def _pp_exprs():
    s = open(SRC).read()
    body = s[s.index("void k_pp(GemmParams p)"):s.index("void k_rb(")]
    end = re.search(r"auto end_step = .*?if \(i \+ (\d) < n\) \{\s*if \(two_w\) wait_vm\(ic<(\d)>\{\}\);"
                    r"\s*else wait_vm\(ic<(\d)>\{\}\);\s*\} else \{\s*wait_vm\(ic<(\d)>\{\}\);", body, re.S)
    dma = re.search(r"if \(g == 3 && ci \+ (\d) < n\) \{\s*issue_wpk\(ci \+ (\d), ci % (\d)\);", body)
    pro = re.search(r"if \(n > 2\) \{\s*issue_wpk\(2, 2\);\s*issue_ws\(2, 2\);\s*if \(two_w\) wait_vm\(ic<(\d)>\{\}\);"
                    r"[^\n]*\n\s*else wait_vm\(ic<(\d)>\{\}\);\s*\} else \{\s*wait_vm\(ic<(\d)>\{\}\);", body, re.S)
    assert end and dma and pro, "ping-pong copy and wait code not found"
    assert end.group(1) == dma.group(1) == dma.group(2), "weights issued and waited at the same distance"
    return {"ahead": int(dma.group(1)), "slots": int(dma.group(3)),
            "end": {2: int(end.group(2)), 1: int(end.group(3)), "last": int(end.group(4))},
            "pro": {2: int(pro.group(1)), 1: int(pro.group(2)), "short": int(pro.group(3))}}


def _replay_pp(kA, kWc, n, ex):
    ops, done = [], 0

    def issue(kind, step, count):
        ops.extend([(kind, step)] * count)

    def wait(c):
        nonlocal done
        done = max(done, len(ops) - c)

    def landed(kind, step):
        return max(k for k, o in enumerate(ops) if o == (kind, step)) < done

    D = ex["ahead"]
    issue("A", 0, 4 * kA)
    for j in range(min(n, D)):
        issue("W", j, kWc)
    wait(ex["pro"][kWc] if n > 2 else ex["pro"]["short"])
    assert landed("A", 0) and landed("W", 0), "prologue: step 0"
    if n > 1:
        assert landed("W", 1), "prologue: weights of step 1, expanded in step 0"
    for i in range(n):
        if i + 1 < n:
            issue("A", i + 1, 4 * kA)
        if i + D < n:
            issue("W", i + D, kWc)
        wait(ex["end"][kWc] if i + D < n else ex["end"]["last"])
        if i + 1 < n:
            assert landed("A", i + 1), f"end of step {i}: activation tile of step {i + 1}"
        if i + 2 < n:
            assert landed("W", i + 2), f"end of step {i}: weights of step {i + 2}"
    # every slot is refilled only after its step was expanded: W(i + D) goes
    # into slot i % slots, the slot of step i, expanded during step i - 1
    assert ex["slots"] == D


def test_ping_pong_copy_waits_cover_every_read():
    ex = _pp_exprs()
    for kA in (1, 2):
        for kWc in (1, 2):
            for n in range(1, 14):
                _replay_pp(kA, kWc, n, ex)


def test_ping_pong_replay_catches_a_short_wait():
    ex = _pp_exprs()
    ex["end"] = {**ex["end"], 2: 3}             # one copy more left in flight than the newest weights
    with pytest.raises(AssertionError, match="end of step"):
        _replay_pp(1, 2, 6, ex)


# Line-staged small-M kernel (nf4_gemv.hip): each wave issues C LDS-direct
# copies per step into kSD private slots, kSD steps ahead; the prologue issues
# the copies of steps 0 .. kSD - 1 after the x and table loads and waits until
# only those copies are in flight; before step ls the wave waits until at most
# the copies of `later` steps are in flight, and after it refills the slot of
# step ls with step ls + kSD.  Step ls reads slot ls % kSD.

GEMV_SRC = os.path.join(ROOT, "nf4_bit_weight_amd", "csrc", "nf4_gemv.hip")


def _ln_exprs():
    s = open(GEMV_SRC).read()
    body = s[s.index("void k_gemv_ln(GemvParams p)"):s.index("size_t gemv_region_bytes(")]
    sd = re.search(r"constexpr int kSD = (\d+);", s)
    c = re.search(r"constexpr int C = (\d+);", body)
    cases = dict(re.findall(r"case (\d+): vm_wait_open<([^>]+)>\(\); break;", body))
    dflt = re.search(r"default: vm_wait_open<([^>]+)>\(\); break;", body)
    later = re.search(r"auto wait_copies = \[&\]\(int ls\) \{\s*const int later = ([^;]+);\s*wait_later\(later\);", body)
    pro = re.search(r"for \(int j = 0; j < kSD; \+\+j\)\s*if \(j < nw\) issue\(j, j\);\s*fence\(\);[^\n]*\n[^\n]*\n"
                    r"\s*wait_later\(([^;]+)\);", body)
    refill = re.search(r"if \(ls \+ kSD < nw\) issue\(ls \+ kSD, slot\);", body)
    issue = body[body.index("auto issue = [&](int ls, int slot)"):body.index("auto wait_later")]
    assert sd and c and cases and dflt and later and pro and refill, "line-staged copy and wait code not found"
    # copies per issue: two packed-line copies, then one scale copy in either form
    assert issue.count("raw_ptr_buffer_load_lds(") == 4 and "if constexpr (NESTED)" in issue
    conv = lambda e: re.sub(r"\(?([^()?]+)\?([^():]+):([^()]+)\)?", r"((\2) if (\1) else (\3))", e)
    return {"kSD": int(sd.group(1)), "C": int(c.group(1)), "cases": {int(k): v for k, v in cases.items()},
            "default": dflt.group(1), "later": conv(later.group(1)), "pro": conv(pro.group(1))}


def _replay_ln(nw, ex):
    kSD, C = ex["kSD"], ex["C"]
    ops, done = [], 0
    issued = set()

    def ev(e, **kw):
        return eval(e, {"__builtins__": {}}, {"kSD": kSD, "C": C, "nw": nw, **kw})

    def vmcnt(later):
        return ev(ex["cases"].get(later, ex["default"]))

    def issue(step):
        assert step not in issued, f"step {step} copied twice"
        issued.add(step)
        ops.extend([("W", step)] * C)

    def wait(c):
        nonlocal done
        done = max(done, len(ops) - c)

    def landed(kind, step):
        return max(k for k, o in enumerate(ops) if o == (kind, step)) < done

    ops.extend([("X", 0)] * 5)                         # x batch and table loads
    for j in range(kSD):
        if j < nw:
            issue(j)
    wait(vmcnt(ev(ex["pro"])))
    assert landed("X", 0), "prologue: x and tables before they are stored"
    slot = {}
    for j in range(min(kSD, nw)):
        slot[j % kSD] = j
    for ls in range(nw):
        wait(vmcnt(ev(ex["later"], ls=ls)))
        assert landed("W", ls), f"before step {ls}: its copies"
        assert slot[ls % kSD] == ls, f"step {ls}: slot holds step {slot[ls % kSD]}"
        if ls + kSD < nw:
            issue(ls + kSD)
            slot[ls % kSD] = ls + kSD
    assert issued == set(range(nw))


def test_line_staged_copy_waits_cover_every_read():
    ex = _ln_exprs()
    for nw in range(0, 70):
        _replay_ln(nw, ex)


@pytest.mark.parametrize("kSD", [2, 3, 4])
def test_line_staged_waits_hold_for_every_slot_count(kSD):
    """The wait code is written for 2 to 4 slots; each count is replayed."""
    ex = {**_ln_exprs(), "kSD": kSD}
    for nw in range(0, 40):
        _replay_ln(nw, ex)


def test_line_staged_replay_catches_a_short_wait():
    ex = _ln_exprs()
    ex["later"] = "(kSD if nw - 1 - ls > kSD else nw - 1 - ls)"   # one step more left in flight
    with pytest.raises(AssertionError, match="before step"):
        _replay_ln(8, ex)
