"""Largest unit the library accepts: 2^31 padded elements.

A unit of 32768 x 65536 (wide) or 65536 x 32768 (tall) bf16 is exactly the
planner's limit.  Every buffer of it passes 2^31 bytes, so any 32-bit
element or byte offset in the planner or the kernels would land elsewhere.
The oracle cannot step a matrix of that size, but this one has a closed
relation to a small one.  The gradient is zero except for three blocks with
disjoint rows and columns, one of them in the far corner (the largest
indices).  Row and column permutations and zero padding commute with every
step of the method: the momentum is elementwise, the Frobenius norm ignores
zeros, and each Newton-Schulz product (Muon blog section 3: A = X X^T,
B = b A + c A^2, X <- a X + B X) keeps the block structure, zero rows and
columns staying exactly zero.  So the blocks of O must match the oracle's O
for the small block-diagonal matrix that assembles the three blocks.  They
are held to the bf16 bar, and the momentum to its bar.  Everything off the
blocks must be exactly zero, in O and in the momentum.  The weights must
follow the decoupled update (Muon README "Usage"): on the blocks as checked
element by element from the GPU's own O, and elsewhere as pure decay, at
sampled positions, bitwise against the oracle's rounding.  The same step
also runs on the bounds-checking debug build, whose every GEMM and
elementwise task checks its tile against the unit's padded sizes and sets a
flag instead of running past them: no flag may be set.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_aware_optimizer_muon_amd as mm
from matrix_aware_optimizer_muon_amd import build
from oracle import muon_oracle as orc
from tests.parity_common import SCALE_NAMES, check_w_update_elementwise, oracle_step, rel_f, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_O = 2e-2
TOL_M = 1e-6

# (row start, column start, rows, cols) of the blocks in the wide unit; the
# tall unit uses the transposed layout.  Odd offsets and sizes leave the
# blocks off every tile boundary; the last one ends at the last row and
# column.
WIDE = (32768, 65536)
BLOCKS_WIDE = [(0, 0, 256, 384), (16421, 40003, 200, 300), (32608, 65088, 160, 448)]


def _layout(orient):
    if orient == "wide":
        return WIDE, BLOCKS_WIDE
    return (WIDE[1], WIDE[0]), [(c0, r0, w, h) for r0, c0, h, w in BLOCKS_WIDE]


@pytest.mark.parametrize("lib", ["release", "debug"])
@pytest.mark.parametrize("orient", ["wide", "tall"])
def test_maximum_unit_block_structured(orient, lib):
    (R, C), blocks = _layout(orient)
    say(f"case: maximum unit {R}x{C} bf16 ({orient}, {lib} build), three blocks of gradient, zeros elsewhere")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([9300, R, C])))
    gblocks = [orc.f64_to_bf16_bits(rng.standard_normal((h, w)) * s)
               for (_, _, h, w), s in zip(blocks, (1.0, 3.0, 0.5))]

    dev = torch.device("cuda")
    G = torch.zeros(R, C, dtype=torch.bfloat16, device=dev)
    for (r0, c0, h, w), gb in zip(blocks, gblocks):
        G[r0:r0 + h, c0:c0 + w] = torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16).to(dev)
    gen = torch.Generator(device=dev).manual_seed(9301)
    W = torch.empty(R, C, dtype=torch.bfloat16, device=dev).normal_(0.0, 0.02, generator=gen)
    M = torch.zeros(R, C, dtype=torch.float32, device=dev)
    O = torch.empty(R, C, dtype=torch.float32, device=dev)

    # weights before the step: the blocks, and sampled positions off them
    # (corners and the last row and column included)
    w0_blocks = [W[r0:r0 + h, c0:c0 + w].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                 for r0, c0, h, w in blocks]
    on_block = lambda i, j: any(r0 <= i < r0 + h and c0 <= j < c0 + w for r0, c0, h, w in blocks)
    cand = [(0, C - 1), (R - 1, 0), (R - 1, C - 1 - 512), (R // 2, C // 2)]
    cand += list(zip(rng.integers(0, R, 4096).tolist(), rng.integers(0, C, 4096).tolist()))
    samples = [(i, j) for i, j in cand if not on_block(i, j)]
    si = torch.tensor([p[0] for p in samples], device=dev)
    sj = torch.tensor([p[1] for p in samples], device=dev)
    w0_samp = W[si, sj].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    hp = mm.default_hparams()
    st = mm.MuonStep([mm.tensor_desc(W, G, M, update_out=O)], hp,
                     library=build.DEBUG_LIB if lib == "debug" else None)
    say(f"  workspace {st.workspace_bytes / 2**30:.1f} GiB; stepping")
    st.step()
    torch.cuda.synchronize()
    assert st.flags() == 0
    st.close()
    del st
    say("  step done; comparing")

    # the oracle on the assembled block-diagonal matrix
    hs, ws = sum(b[2] for b in blocks), sum(b[3] for b in blocks)
    assert (hs > ws) == (R > C), "the small matrix must take the same side as the unit"
    Gs = np.zeros((hs, ws), np.uint16)
    offs, ro, co = [], 0, 0
    for (_, _, h, w), gb in zip(blocks, gblocks):
        Gs[ro:ro + h, co:co + w] = gb
        offs.append((ro, co))
        ro, co = ro + h, co + w
    ref = oracle_step(np.zeros((hs, ws), np.uint16), Gs, np.zeros((hs, ws)), "bf16", hp)

    o_blk, m_blk = np.zeros((hs, ws)), np.zeros((hs, ws))
    for (r0, c0, h, w), (ro, co) in zip(blocks, offs):
        o_blk[ro:ro + h, co:co + w] = O[r0:r0 + h, c0:c0 + w].cpu().numpy()
        m_blk[ro:ro + h, co:co + w] = M[r0:r0 + h, c0:c0 + w].cpu().numpy()
    e_o, e_m = rel_f(o_blk, ref["O"]), rel_f(m_blk, ref["M"])

    # fused update on the blocks, from the GPU's own O, with the unit's scale
    scale = orc.shape_scale(R, C, SCALE_NAMES[hp.scale_mode])
    worst = 0.0
    for (r0, c0, h, w), w0b in zip(blocks, w0_blocks):
        w1b = W[r0:r0 + h, c0:c0 + w].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        ulp, _ = check_w_update_elementwise(w1b, w0b, O[r0:r0 + h, c0:c0 + w].cpu().numpy(), float(hp.lr),
                                            float(hp.weight_decay), [scale] * h)
        worst = max(worst, ulp)
    # pure decay elsewhere: one rounding of W - lr*wd*W
    w1_samp = W[si, sj].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    decay = orc.f64_to_bf16_bits(orc.apply_update(orc.bf16_bits_to_f64(w0_samp), np.zeros(len(samples)),
                                                  float(hp.lr), float(hp.weight_decay), scale))
    decay_bad = int(np.count_nonzero(w1_samp != decay))

    # everything off the blocks is exactly zero in O and in the momentum
    for r0, c0, h, w in blocks:
        O[r0:r0 + h, c0:c0 + w] = 0.0
        M[r0:r0 + h, c0:c0 + w] = 0.0
    nz_o, nz_m = int(torch.count_nonzero(O)), int(torch.count_nonzero(M))
    say(f"  O {e_o:.2e}  M {e_m:.2e}  fused update max {worst:.2f} of bound  "
        f"decay samples off by a bit: {decay_bad} of {len(samples)}  nonzeros off the blocks: O {nz_o}, M {nz_m}")
    del G, W, M, O
    torch.cuda.empty_cache()
    assert e_o <= TOL_O and e_m <= TOL_M
    assert worst <= 1.0 and decay_bad == 0
    assert nz_o == 0 and nz_m == 0
