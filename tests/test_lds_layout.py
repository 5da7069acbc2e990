"""The LDS block images (csrc/xfa_stage.h) without a GPU: a host-only build of
the header reports each bf16 geometry (slots per row P, the row map phys, the
DMA strip counts), and these tests check the properties the kernels rely on
against a model of the LDS banks: 64 banks of 4 bytes, a 16-byte read served
16 lanes per cycle, an 8-byte (transpose) read 32 lanes per cycle.  On the
GPU the same property shows as SQ_LDS_BANK_CONFLICT = 0 in every kernel."""

import os
import subprocess

import pytest

from transformer_attention_xfa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_attention_xfa_amd", "csrc")
HDS = (16, 32, 64, 128)

PROBE = r"""
#include <cstdio>
#include "xfa_stage.h"
using namespace xfa;
template <int HD> void show() {
  using G = BlockGeo<bf16, HD, 4>;
  using K = Dma<bf16, HD, 4, 2, true>;    // key workgroups: Q, dO, L and D
  using F = Dma<bf16, HD, 4, 2, false>;   // forward and query workgroups: two tensors
  std::printf("%d %d %d %d %d %d %d %d %d", HD, G::HDP, G::P, G::CPR, K::NI, K::NS, K::NPW, F::NS, F::NPW);
  for (int r = 0; r < G::NB; ++r) std::printf(" %d", G::phys(r));
  std::printf("\n");
}
int main() { show<16>(); show<32>(); show<64>(); show<128>(); return 0; }
"""


@pytest.fixture(scope="module")
def geo(tmp_path_factory):
    d = tmp_path_factory.mktemp("lds")
    src, exe = d / "probe.hip", d / "probe"
    src.write_text(PROBE)
    cmd = [B.hipcc(), "-x", "hip", "--offload-host-only", "-std=c++17", "-I", CSRC, "-I",
           os.path.join(ROOT, "include"), str(src), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    g = {}
    for line in out.strip().splitlines():
        v = [int(x) for x in line.split()]
        hd, hdp, P, cpr, ni, kns, knpw, fns, fnpw = v[:9]
        g[hd] = dict(HDP=hdp, P=P, CPR=cpr, NI=ni, key_NS=kns, key_NPW=knpw, fwd_NS=fns, fwd_NPW=fnpw, phys=v[9:])
    return g


def slot(g, r, ch):
    return g["phys"][r] * g["P"] + ch


def worst_bank_use(addrs, width):
    """Most distinct dwords any one bank serves for these lane addresses."""
    banks = {}
    for a in addrs:
        for w in range(width // 4):
            dw = a // 4 + w
            banks.setdefault(dw % 64, set()).add(dw)
    return max(len(s) for s in banks.values())


@pytest.mark.parametrize("hd", HDS)
def test_rows_fit_their_strips_without_overlap(geo, hd):
    g = geo[hd]
    assert sorted(g["phys"]) == list(range(32))
    assert all(g["phys"][g["phys"][r]] == r for r in range(32))      # its own inverse
    slots = {slot(g, r, ch) for r in range(32) for ch in range(g["HDP"] // 8)}
    assert len(slots) == 32 * g["HDP"] // 8
    assert max(slots) < 64 * g["NI"] and g["P"] >= g["HDP"] // 8


@pytest.mark.parametrize("hd", HDS)
def test_natural_reads_are_conflict_free(geo, hd):
    # lane l reads the 16 bytes at block row l % 32, slot 2c + l / 32
    g = geo[hd]
    for c in range(max(1, hd // 16)):
        addrs = [16 * slot(g, l & 31, 2 * c + (l >> 5)) for l in range(64)]
        for ph in range(4):
            assert worst_bank_use(addrs[16 * ph:16 * ph + 16], 16) == 1, (hd, c, ph)


@pytest.mark.parametrize("hd", HDS)
def test_transpose_reads_are_conflict_free(geo, hd):
    # ds_read_b64_tr_b16: lane l (t = l % 16, nb = bit 4, h = l / 32) reads 8
    # bytes at block row 4h + t/4 (+8 for the second read of an operand, +16u)
    # and byte 64d + 32nb + 8(t % 4) of that row
    g = geo[hd]
    for u in range(2):
        for d in range(g["HDP"] // 32):
            for second in range(2):
                addrs = []
                for l in range(64):
                    t, nb, h = l & 15, (l >> 4) & 1, l >> 5
                    k = 4 * h + (t >> 2) + 8 * second + 16 * u
                    byte = 64 * d + 32 * nb + 8 * (t & 3)
                    addrs.append(16 * slot(g, k, byte // 16) + byte % 16)
                for ph in range(2):
                    assert worst_bank_use(addrs[32 * ph:32 * ph + 32], 8) == 1, (hd, u, d, second, ph)


@pytest.mark.parametrize("hd", HDS)
def test_read_offsets_are_per_lane_base_plus_constant(geo, hd):
    # the kernels read rows r + 8 (r mod 16 < 8) and r + 16 at fixed offsets
    g = geo[hd]
    ph = g["phys"]
    assert {ph[k + 8] - ph[k] for k in list(range(8)) + list(range(16, 24))} == {2}
    assert {ph[k + 16] - ph[k] for k in range(16)} == {16}


def test_key_workgroup_waves_issue_five_strips_per_block(geo):
    # hd 128: nine strips per tensor image; with L and D the four waves of a
    # key workgroup issue five each (the padded 20-slot rows took six)
    g = geo[128]
    assert g["P"] == 17 and g["NI"] == 9
    assert (g["key_NS"], g["key_NPW"]) == (20, 5)
    assert (g["fwd_NS"], g["fwd_NPW"]) == (18, 5)
