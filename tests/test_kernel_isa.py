"""Static checks of the attention kernels' gfx950 assembly, compiled here with the
library's own flags (no GPU needed).

An MFMA reads its A and B operands across all 64 lanes of the wave, so it must never
run while the exec mask is narrowed by a divergent branch: the inactive lanes' operand
rows would be dropped.  The compiler is free to move instructions whose results are only
used inside such a branch into it (it once moved the last tile's P^V MFMAs into the
epilogue's `row < N_q` branch), so every build is checked: a forward dataflow over each
kernel's control-flow graph marks where the mask may be narrowed (after
s_and_saveexec / s_or_saveexec, until exec is restored with s_or_b64 / s_mov_b64), and
no MFMA may be reachable in such a state.  The check itself is pinned by a synthetic
listing that it must flag."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "mxfp4_bit_attention_amd"))


def mfma_under_narrowed_exec(asm: str) -> dict:
    """{kernel symbol: number of MFMAs reachable with a narrowed exec mask}."""
    lines = asm.split("\n")
    out = {}
    starts = [k for k, l in enumerate(lines) if re.match(r"^_Z\w*k_attn\w*:", l)]
    for s in starts:
        e = next(k for k in range(s, len(lines)) if "s_endpgm" in lines[k])
        blocks, cur = [], ("entry", [])
        for l in lines[s + 1:e + 1]:
            t = l.strip()
            if not t or t.startswith(";"):
                continue
            m = re.match(r"^(\.LBB\d+_\d+):", t)
            if m:
                blocks.append(cur)
                cur = (m.group(1), [])
                continue
            if t.startswith("."):
                continue
            cur[1].append(t)
        blocks.append(cur)
        idx = {b[0]: i for i, b in enumerate(blocks)}
        entry = [False] * len(blocks)

        def walk(i, mark):
            state, bad, fall = entry[i], 0, True
            for t in blocks[i][1]:
                tk = t.split()
                op = tk[0]
                dst = tk[1].rstrip(",") if len(tk) > 1 else ""
                if op in ("s_and_saveexec_b64", "s_or_saveexec_b64"):
                    state = True
                elif op in ("s_or_b64", "s_mov_b64") and dst == "exec":
                    state = False
                if op.startswith("v_mfma") and state:
                    bad += 1
                if (op.startswith("s_cbranch") or op == "s_branch") and tk[1] in idx:
                    mark(idx[tk[1]], state)
                if op in ("s_branch", "s_endpgm"):
                    fall = False
            if fall and i + 1 < len(blocks):
                mark(i + 1, state)
            return bad

        changed = [True]

        def mark(j, st):
            if st and not entry[j]:
                entry[j] = True
                changed[0] = True

        while changed[0]:
            changed[0] = False
            for i in range(len(blocks)):
                walk(i, mark)
        out[lines[s].split(":")[0]] = sum(walk(i, lambda j, st: None) for i in range(len(blocks)))
    return out


def test_checker_flags_an_mfma_inside_a_divergent_branch():
    asm = "\n".join([
        "_ZN6mxattn6k_attnILi128EEEvv:",
        "  v_cmp_gt_i32_e32 vcc, s0, v1",
        "  v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:19], v[20:23], v[0:15], v24, v25",
        "  s_and_saveexec_b64 s[2:3], vcc",
        "  s_cbranch_execz .LBB0_2",
        ".LBB0_1:",
        "  v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:19], v[20:23], v[0:15], v24, v25",
        "  global_store_dwordx4 v[30:31], v[0:3], off",
        ".LBB0_2:",
        "  s_or_b64 exec, exec, s[2:3]",
        "  v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:19], v[20:23], v[0:15], v24, v25",
        "  s_endpgm",
    ])
    assert list(mfma_under_narrowed_exec(asm).values()) == [1]


def test_no_attention_mfma_runs_under_a_narrowed_exec_mask(tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    import build as b
    src = os.path.join(b.CSRC, "attention.hip")
    out = str(tmp_path / "attention.s")
    cmd = [b.hipcc(), *b.common_flags(), *b.EXTRA_FLAGS.get("attention.hip", []), "--cuda-device-only", "-S",
           src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    res = mfma_under_narrowed_exec(open(out).read())
    assert len(res) >= 8  # every d x PNQ x dump x scale-layout instantiation
    assert all(n == 0 for n in res.values()), res
