"""The matrix-core operand layouts the bfloat16 kernels assume, as a numpy model (CPU only), and a
guard on the built library against one instruction pairing that gives wrong results on gfx950.

Layouts assumed by csrc/prefill_mfma.hip and csrc/backward.hip (lane l of a 64-wide wavefront,
g = l // 16, i = l % 16):
  * 16x16x16 bf16 (D = A B + C): lane holds A[i][4g + r] and B[4g + r][i], r = 0..3;
  * 16x16x32 bf16: lane holds A[i][8g + r] and B[8g + r][i], r = 0..7;
  * both: lane holds D[4g + r][i], r = 0..3.
These were checked on an MI355X with exactly representable inputs (small integers): each form, the
16x16x32 form's two k-halves, and a 16x16x16 accumulator reused as the next A operand (A' = D^T) gave
the exact products.  The model below builds the fragments from those rules and checks the identities
the kernels rely on: two k-halves carrying hi and lo terms against a duplicated operand sum to
(hi + lo) B; an accumulator's four elements reused as an A operand act as D^T; and the readout's
state-in-accumulator operand, paired with phi(sQ) stored in the kernels' slot order, gives phi(sQ) S.

The guard: a 16x16x32 bf16 MFMA followed at once by a 16x16x16 bf16 MFMA that takes the first one's
result as its accumulator gave wrong sums on gfx950 (the compiler issued them back to back, one cycle
apart; with 10 or 17 cycles of other instructions between them the sums were exact, and so were the
reverse order at 7 or 8 cycles and two dependent 16x16x32s).  That pairing explains the wrong dk of an
earlier fused backward variant.  The guard flags any MFMA reading the result of an MFMA of another
opcode less than 10 cycles later; no kernel may contain one.
"""

import glob
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import recurrent_state_amd as rs

LANES = 64


def frag_a(A, k):
    """A [16, K] -> per-lane fragments [64, k] of a 16x16xK form (k = K / 4 values per lane)."""
    return np.array([[A[l % 16, k * (l // 16) + r] for r in range(k)] for l in range(LANES)])


def frag_b(B, k):
    return np.array([[B[k * (l // 16) + r, l % 16] for r in range(k)] for l in range(LANES)])


def mfma(fa, fb, fc=None):
    """The product of fragments under the assumed layouts: rebuild A and B, multiply, fragment D."""
    k = fa.shape[1]
    A = np.zeros((16, 4 * k))
    B = np.zeros((4 * k, 16))
    for l in range(LANES):
        for r in range(k):
            A[l % 16, k * (l // 16) + r] = fa[l, r]
            B[k * (l // 16) + r, l % 16] = fb[l, r]
    D = A @ B
    out = np.array([[D[4 * (l // 16) + r, l % 16] for r in range(4)] for l in range(LANES)])
    return out if fc is None else out + fc


def unfrag_d(fd):
    D = np.zeros((16, 16))
    for l in range(LANES):
        for r in range(4):
            D[4 * (l // 16) + r, l % 16] = fd[l, r]
    return D


def test_k_halves_carry_two_terms():
    rng = np.random.default_rng(1)
    hi, lo = rng.standard_normal((16, 16)), rng.standard_normal((16, 16))
    B = rng.standard_normal((16, 16))
    # lane fragments of the 16-deep operands, concatenated as the two halves of one 32-deep operand
    fa = np.concatenate([frag_a(hi, 4), frag_a(lo, 4)], axis=1)
    fb = np.concatenate([frag_b(B, 4), frag_b(B, 4)], axis=1)
    np.testing.assert_allclose(unfrag_d(mfma(fa, fb)), (hi + lo) @ B, rtol=1e-12, atol=1e-12)
    # a planted mistake: the halves of B swapped with another operand's break the identity
    fb_bad = np.concatenate([frag_b(B, 4), frag_b(B.T, 4)], axis=1)
    assert not np.allclose(unfrag_d(mfma(fa, fb_bad)), (hi + lo) @ B)


def test_accumulator_reused_as_an_a_operand_is_transposed():
    rng = np.random.default_rng(2)
    A, B, B2 = rng.standard_normal((16, 16)), rng.standard_normal((16, 16)), rng.standard_normal((16, 16))
    d1 = mfma(frag_a(A, 4), frag_b(B, 4))  # lane holds D1[4g + r][i]
    # those four values are the lane's A operand: A'[i][4g + r] = D1[4g + r][i]
    np.testing.assert_allclose(unfrag_d(mfma(d1, frag_b(B2, 4))), (A @ B).T @ B2, rtol=1e-12, atol=1e-12)


def slot_feature(s):
    """Feature at position s of a phi(sQ) row in the bf16 readout: in each 32-feature block, lane group g
    holds features 4g..4g+3 and 16+4g..16+4g+3 (the rows its accumulator elements of two 16-row state
    tiles cover)."""
    kb, r32 = divmod(s, 32)
    g, r = divmod(r32, 8)
    return 32 * kb + (4 * g + r if r < 4 else 16 + 4 * g + r - 4)


def test_readout_from_state_accumulators():
    # S^T tiles (value columns x features) live in accumulators: tile t, lane (c = i, g) holds
    # S^T[c][16 t + 4 g + r].  Two consecutive tiles' four elements form the lane's eight-value A operand
    # of a 32-deep product over features; phi(sQ) rows are stored in slot order, so the B operand's k
    # index s stands for feature slot_feature(s).  The result must be S^T phi(sQ)^T.
    rng = np.random.default_rng(3)
    W, T = 64, 16  # two 32-feature blocks, one 16-token tile
    ST = rng.standard_normal((16, W))  # 16 value columns
    phiq = rng.standard_normal((T, W))
    out = np.zeros((LANES, 4))
    for kb in range(W // 32):
        acc = [np.array([[ST[l % 16, 32 * kb + 16 * h + 4 * (l // 16) + r] for r in range(4)] for l in range(LANES)])
               for h in range(2)]
        fa = np.concatenate(acc, axis=1)
        Bperm = np.array([[phiq[t, slot_feature(32 * kb + s)] for t in range(T)] for s in range(32)])
        out = mfma(fa, frag_b(Bperm, 8), out)
    np.testing.assert_allclose(unfrag_d(out), ST @ phiq.T, rtol=1e-12, atol=1e-12)
    # the natural feature order in the B operand would be wrong
    bad = np.zeros((LANES, 4))
    for kb in range(W // 32):
        acc = [np.array([[ST[l % 16, 32 * kb + 16 * h + 4 * (l // 16) + r] for r in range(4)] for l in range(LANES)])
               for h in range(2)]
        bad = mfma(np.concatenate(acc, axis=1), frag_b(phiq[:, 32 * kb: 32 * kb + 32].T, 8), bad)
    assert not np.allclose(unfrag_d(bad), ST @ phiq.T)


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok) or re.match(r"([va])(\d+)$", tok)
    if not m:
        return set()
    a = int(m.group(2))
    b = int(m.group(3)) if m.lastindex == 3 else a
    return {(m.group(1), r) for r in range(a, b + 1)}


def mixed_mfma_chains(lines, min_gap=10):
    """(index, first opcode, second opcode, gap) for every MFMA read (A, B or C operand) of an MFMA result
    of a different opcode with fewer than `min_gap` cycles of other instructions between them."""
    insts = []
    for line in lines:
        t = line.split("//")[0].split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            insts.append(None if t.startswith(".") or t.endswith(":") else "")
            continue
        insts.append(t)
    found = []
    for i, t in enumerate(insts):
        if not t or not t.startswith("v_mfma"):
            continue
        op, rest = t.split(None, 1)
        dst = _regs(rest.split(",")[0].strip())
        gap = 0
        for j in range(i + 1, min(i + 24, len(insts))):
            u = insts[j]
            if u is None:  # a label: control may arrive from elsewhere
                break
            if not u:
                continue
            if u.startswith("s_nop"):
                gap += int(u.split()[1], 0) + 1
                continue
            if u.startswith("v_mfma"):
                op2, rest2 = u.split(None, 1)
                srcs = set().union(*(_regs(x.strip()) for x in rest2.split(",")[1:4]))
                if srcs & dst:
                    if op2 != op and gap < min_gap:
                        found.append((i, op, op2, gap))
                    break
            if " " in u and dst & _regs(u.split(None, 1)[1].split(",")[0].strip()):
                break  # the result was overwritten
            gap += 1
            if gap >= min_gap:
                break
    return found


def test_scanner_flags_the_pairing():
    bad = ["v_mfma_f32_16x16x32_bf16 v[2:5], v[2:5], v[10:13], 0",
           "v_mfma_f32_16x16x16_bf16 v[2:5], v[14:15], v[10:11], v[2:5]"]
    assert mixed_mfma_chains(bad)
    spaced = [bad[0], "s_nop 7", "s_nop 7", bad[1]]
    assert not mixed_mfma_chains(spaced)
    same = [bad[0], "v_mfma_f32_16x16x32_bf16 v[2:5], v[6:9], v[10:13], v[2:5]"]
    assert not mixed_mfma_chains(same)


OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.mark.skipif(not (os.path.exists(rs.LIB_PATH) and os.path.exists(OBJDUMP)), reason="library or objdump missing")
def test_built_library_has_no_mixed_mfma_chain():
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "lib.so")
        shutil.copy(rs.LIB_PATH, lib)
        subprocess.run([OBJDUMP, "--offloading", lib], cwd=d, check=True, capture_output=True)
        objs = sorted(glob.glob(os.path.join(d, "lib.so.*gfx950")))
        assert objs, "no gfx950 code object in the library"
        total = 0
        for obj in objs:
            out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", obj], check=True, capture_output=True, text=True).stdout
            lines = out.split("\n")
            total += sum(1 for line in lines if "v_mfma" in line)
            bad = mixed_mfma_chains(lines)
            assert not bad, f"{os.path.basename(obj)}: {bad[:3]}"
        assert total > 1000  # the matrix-core kernels are there
