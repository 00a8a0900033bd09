"""The batched round's host logic (include/gptq.h, gptq_round_plan / gptq_round_slot_size) and
its schedule in check mode, on the CPU: widest-first order, concurrency capped by the workspace
(page "cortiq-cli 0.8.45 src/gptq.rs", run_quantize_gptq_tiled and fold_concurrency), the
slot's size from the per-call workspace queries, the C structures' layout as the binding sees
it, and every call of a config-sized round inside its buffers."""
import ctypes
import os
import subprocess

import pytest

import post_weight_quantization_amd as pwq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE, STRIDE = 1 << 44, 1 << 38
_next = [0]


def fake():
    _next[0] += 1
    return BASE + _next[0] * STRIDE


def group(n, rows=(), codec="q4tp", ldh=None, precision="auto", lam=0.01):
    ms = (pwq.RoundMember * max(len(rows), 1))()
    for k, r in enumerate(rows):
        ms[k] = pwq.RoundMember(fake(), r, pwq.CODEC[codec], 0, fake(), fake(), fake(), fake(), fake())
    g = pwq.RoundGroup(fake(), n, n if ldh is None else ldh, lam, pwq.FOLD_PRECISION[precision],
                       len(rows), ms, fake(), fake(), pwq.FoldReport(), 0, 0)
    return g, ms


def array(specs):
    keep = [group(*s[:2], **(s[2] if len(s) > 2 else {})) for s in specs]
    arr = (pwq.RoundGroup * len(keep))(*[g for g, _ in keep])
    return arr, keep


@pytest.fixture(scope="module")
def lib():
    return pwq.load()


def plan(lib, arr, ws, conc):
    order = (ctypes.c_int32 * len(arr))()
    c = ctypes.c_int32(-1)
    st = lib.gptq_round_plan(arr, len(arr), ws, conc, order, ctypes.byref(c))
    return st, list(order), c.value


def a256(x):
    return (x + 255) // 256 * 256


def test_structures_match_the_header(tmp_path):
    """sizeof / offsetof of gptq_member, gptq_group and gptq_fold_report as a C compiler lays
    them out equal the binding's ctypes structures."""
    src = str(tmp_path / "abi_probe.c")
    exe = str(tmp_path / "abi_probe")
    fields = {"gptq_member": [f for f, _ in pwq.RoundMember._fields_],
              "gptq_group": [f if f != "lam" else "lambda" for f, _ in pwq.RoundGroup._fields_],
              "gptq_fold_report": [f for f, _ in pwq.FoldReport._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gptq.h"', "int main(void) {"]
    for t, fs in fields.items():
        lines.append(f'printf("%zu\\n", sizeof({t}));')
        lines += [f'printf("%zu\\n", offsetof({t}, {f}));' for f in fs]
    lines.append("return 0; }")
    open(src, "w").write("\n".join(lines))
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
    got = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = []
    for cls in (pwq.RoundMember, pwq.RoundGroup, pwq.FoldReport):
        want.append(ctypes.sizeof(cls))
        want += [getattr(cls, f).offset for f, _ in cls._fields_]
    assert got == want


def test_widest_first_order(lib):
    arr, keep = array([(4096, (4096,)), (17408, (5120,)), (4096, (4096, 1024)), (8192, (2048,)),
                       (17408, (5120,)), (4096, (4096,))])
    st, order, c = plan(lib, arr, 1 << 50, 0)
    assert st == pwq.GPTQ_OK
    assert order == [1, 4, 3, 2, 0, 5]  # n, then member rows, then index
    assert c == 2  # gangs: groups 1 and 4, groups 0 and 5 (2 has another member)


def test_gangs_and_threads(lib):
    """Consecutive groups of the plan's order with the same shape (n, precision, damping,
    members' rows and codecs; not f64) form gangs of at most the cap (16 by default), which use
    one slot each; a round without a gang of two runs on threads, 4 at a time by default."""
    arr, keep = array([(n, (64,)) for n in (256, 512, 768, 1024, 1280, 1536)])
    assert plan(lib, arr, 1 << 50, 0)[2] == 4
    assert plan(lib, arr, 1 << 50, 6)[2] == 6
    arr, keep = array([(512, (64,))] * 20)
    assert plan(lib, arr, 1 << 50, 0)[2] == 16
    assert plan(lib, arr, 1 << 50, 7)[2] == 7
    arr, keep = array([(512, (64,)), (512, (64,), {"lam": 1e-3}), (512, (64,), {"codec": "q2tp"}),
                       (512, (64,), {"precision": "f64"}), (512, (64,), {"precision": "f64"})])
    assert plan(lib, arr, 1 << 50, 0)[2] == 4  # no two of them alike (f64 groups never gang)


def test_concurrency_is_capped_by_the_workspace(lib):
    """fold_concurrency's rule on the device: the groups at once are the workspace over one
    slot, at least one, at most the cap and the number of groups."""
    arr, keep = array([(4096, (4096,))] * 11)
    slot = lib.gptq_round_slot_size(arr, 11)
    assert plan(lib, arr, slot - 1, 0)[0] == pwq.GPTQ_EWORKSPACE
    assert plan(lib, arr, slot, 0)[2] == 1
    assert plan(lib, arr, 3 * slot + slot // 2, 0)[2] == 3
    assert plan(lib, arr, 100 * slot, 0)[2] == 11  # one gang
    assert plan(lib, arr, 100 * slot, 16)[2] == 11
    assert plan(lib, arr, 100 * slot, 2)[2] == 2


@pytest.mark.parametrize("precision", ["auto", "f32", "f64"])
def test_slot_size_from_the_call_workspaces(lib, precision):
    """A slot is U, hdiag and dead plus the larger of the fold's workspace and a member's area
    (they share it), each part 256-byte aligned; the maximum over the groups.  A member's area
    is the sweep's workspace (working copy, two residual panels of 512 columns) followed by its
    outputs (lo / step, TAB, codes, rungs, scales), where a gang stages them."""
    specs = [(4096, (4096, 8192), {"precision": precision}), (1000, (), {"precision": precision}),
             (96, (40000,), {"precision": precision})]
    arr, keep = array(specs)
    sizes = []
    for n, rows, _ in specs:
        work = lib.gptq_fold_workspace_size_ex(n, pwq.FOLD_PRECISION[precision])
        for r in rows:
            sweep = lib.gptq_sweep_workspace_size(r, n)
            assert sweep == a256(4 * r * n) + 2 * a256(4 * r * 512)
            outputs = (a256(4 * r * 2) + a256(4 * r * 32) + a256(r * n // 2) + a256(r * n // 32)
                       + a256(4 * r * n // 32))
            work = max(work, sweep + outputs)
        sizes.append(a256(4 * n * n) + a256(4 * n) + a256(n) + a256(work))
    assert lib.gptq_round_slot_size(arr, 3) == max(sizes)
    assert lib.gptq_round_slot_size(arr, 0) == 0


@pytest.mark.parametrize("bad", [
    {"n": 0}, {"ldh": 100}, {"ldh": -2}, {"precision": 5}, {"codec": 7}, {"rows": 0},
    {"n_mod_32": True}, {"null_member": True}, {"null_out": True}])
def test_invalid_groups_are_refused(lib, bad):
    g, ms = group(256, (64,))
    if "n" in bad:
        g.n = bad["n"]
    if "ldh" in bad:
        g.ldh = bad["ldh"]
    if "precision" in bad:
        g.precision = bad["precision"]
    if "codec" in bad:
        ms[0].codec = bad["codec"]
    if "rows" in bad:
        ms[0].rows = bad["rows"]
    if "n_mod_32" in bad:
        g.n, g.ldh = 250, 250
    if "null_member" in bad:
        g.member = ctypes.POINTER(pwq.RoundMember)()
    if "null_out" in bad:
        ms[0].scale = None
    arr = (pwq.RoundGroup * 1)(g)
    assert lib.gptq_round_slot_size(arr, 1) == 0
    assert plan(lib, arr, 1 << 50, 0)[0] == pwq.GPTQ_EINVAL
    with pwq.check_mode():
        assert lib.gptq_round(arr, 1, ctypes.c_void_p(BASE), 1 << 50, 0, None) == pwq.GPTQ_EINVAL


def test_packed_and_group_without_members(lib):
    arr, keep = array([(300, (), {"ldh": pwq.GPTQ_PACKED_UPPER}), (64, (16,), {"ldh": -1})])
    assert plan(lib, arr, 1 << 50, 0)[0] == pwq.GPTQ_OK


@pytest.mark.parametrize("specs,conc", [
    ([(4096, (4096,))] * 11, 4),
    ([(4096, (4096,))] * 11, 11),
    ([(4096, (4096,))] * 11, 16),
    ([(1184, (77, 300), {"lam": 1e-5})] * 3 + [(1184, (77, 300), {"lam": 1e-5, "codec": "q2tp"})] * 2, 5),
    ([(640, (96,), {"ldh": pwq.GPTQ_PACKED_UPPER}), (640, (96,)), (640, (96,), {"ldh": 700}),
      (2048, (512,), {"precision": "f32"}), (2048, (512,), {"precision": "f32"}), (256, (33,))], 4),
    ([(17408, (5120,)), (4096, (4096, 1024), {"codec": "q2tp"}), (8192, (2048,), {"precision": "f64"}),
      (5120, (512,), {"ldh": pwq.GPTQ_PACKED_UPPER}), (96, ())], 3),
    ([(256, (512,))] * 5, 1),
])
def test_round_schedule_in_check_mode(lib, specs, conc):
    """Every call of the round (fold, ladders, sweeps, on each slot's stream) checked: its
    accesses inside the caller's buffers and its slot of the workspace."""
    arr, keep = array(specs)
    slot = lib.gptq_round_slot_size(arr, len(arr))
    with pwq.check_mode():
        st = lib.gptq_round(arr, len(arr), ctypes.c_void_p(BASE), slot * conc, 0, None)
    assert st == pwq.GPTQ_OK, pwq.check_message()
    assert all(g.status == pwq.GPTQ_OK for g in arr)
    # A workspace one byte short of the slots it names runs one slot fewer, or not at all.
    with pwq.check_mode():
        st = lib.gptq_round(arr, len(arr), ctypes.c_void_p(BASE), slot * conc - 1, 0, None)
    assert st == (pwq.GPTQ_OK if conc > 1 else pwq.GPTQ_EWORKSPACE), pwq.check_message()
    # A misaligned workspace is refused.
    with pwq.check_mode():
        assert lib.gptq_round(arr, len(arr), ctypes.c_void_p(BASE + 16), slot * conc, 0,
                              None) == pwq.GPTQ_EINVAL


def test_gang_schedule_without_hdiag_or_dead_outputs(lib):
    """A gang whose groups give no hdiag or dead buffers (optional outputs): their copies out of
    the slots are skipped, and the schedule checks."""
    arr, keep = array([(512, (64,))] * 5)
    for k in (1, 3):
        arr[k].hdiag = None
        arr[k].dead = None
    slot = lib.gptq_round_slot_size(arr, len(arr))
    with pwq.check_mode():
        st = lib.gptq_round(arr, len(arr), ctypes.c_void_p(BASE), slot * 5, 0, None)
    assert st == pwq.GPTQ_OK, pwq.check_message()
