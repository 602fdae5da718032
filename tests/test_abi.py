"""CPU-side tests of the C-ABI library: it loads, exports every symbol the
header declares, its C++ contract builder matches the contract oracle bit
for bit, its validator accepts valid tables and rejects corrupted ones, and
bad arguments return the documented status without touching the GPU."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import mixture_experts_routed_grouped_amd as R
import workloads
from oracle import contract as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "routed_moe.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"RMOE_API\s+[\w\s\*]+?\b(rmoe_\w+)\s*\(", text)


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 11
    L = ctypes.CDLL(R.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(R._SIGS), "binding and header disagree"


def _compare_tables(lib_c, orc):
    for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx",
                "order", "padded_row_of_pair", "compact_pos_of_pair"]:
        assert np.asarray(lib_c[key]).tolist() == list(orc[key]), key
    assert lib_c["num_blocks_m"] == orc["num_blocks_m"]


@pytest.mark.parametrize("seed", range(10))
def test_contract_matches_oracle_random(seed):
    rng = np.random.default_rng(500 + seed)
    E = int(rng.integers(1, 40))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(0, 1500))
    cfg = workloads.Config("r", T, E, k, 128, 128, routing="zipf" if seed % 2 else "uniform",
                           zipf_s=1.2, seed=seed)
    ids = workloads.draw_routing(cfg)
    _compare_tables(R.build_contract(ids, E), C.build_contract(ids.tolist(), E))


def test_contract_matches_oracle_workloads():
    for name, cfg in workloads.CONFIGS.items():
        ids = workloads.draw_routing(cfg)
        _compare_tables(R.build_contract(ids, cfg.experts), C.build_contract(ids.tolist(), cfg.experts))


def test_contract_handworked():
    with open(os.path.join(ROOT, "tests", "golden", "contract_handworked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        ids = workloads.routing_from_counts(case["counts"], seed=1)
        c = R.build_contract(ids, case["experts"])
        for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx"]:
            assert c[key].tolist() == case[key]
        assert c["num_blocks_m"] == case["num_blocks_m"]


def test_validate_contract():
    ids = workloads.draw_routing(workloads.CONFIGS["fine"])
    c = R.build_contract(ids, 64)
    args = [c["group_sizes"], c["group_offsets"], c["group_padded_offsets"], c["group_idx_for_bx"]]
    tail = (64, c["num_blocks_m"], c["total_padded_tokens"], c["pairs"])
    assert R.validate_contract(*args, *tail) == 0
    bad = [a.copy() for a in args]
    bad[3][5] += 1                                        # a block mapped to the wrong expert
    assert R.validate_contract(*bad, *tail) == -5
    bad = [a.copy() for a in args]
    bad[2][3:] += 128                                     # padded span without the slack rule
    assert R.validate_contract(*bad, *tail) == -5
    bad = [a.copy() for a in args]
    bad[1][7] -= 1                                        # offsets inconsistent with sizes
    assert R.validate_contract(*bad, *tail) == -5
    assert R.validate_contract(*args, 64, c["num_blocks_m"], c["total_padded_tokens"] - 128,
                               c["pairs"]) == -5          # padded buffer too short
    assert R.validate_contract(*args, 64, c["num_blocks_m"], c["total_padded_tokens"],
                               c["pairs"] + 1) == -5


def test_build_contract_errors():
    L = R.lib()
    ids = np.array([[0, 4]], np.int32)                    # id out of range
    with pytest.raises(R.RmoeError):
        R.build_contract(ids, 4)
    gs = np.zeros(4, np.int32)
    go = np.zeros(5, np.int32)
    gpo = np.zeros(5, np.int32)
    gidx = np.zeros(1, np.int32)
    M = np.zeros(1, np.int32)
    ids = np.zeros((300, 1), np.int32)
    p = lambda a: ctypes.c_void_p(a.ctypes.data)
    st = L.rmoe_build_contract(p(ids), 300, 1, 4, p(gs), p(go), p(gpo), p(gidx), 1, p(M), None,
                               None, None)
    assert st == -6                                       # capacity too small
    # 2^24 experts: 128 * num_blocks_m no longer fits the int32 padded offsets
    st = L.rmoe_build_contract(p(ids), 300, 1, 1 << 24, p(gs), p(go), p(gpo), p(gidx), 1 << 30,
                               p(M), None, None, None)
    assert st == -1


def test_argument_errors_without_gpu():
    """Argument checks run before any HIP call, so they are testable here."""
    L = R.lib()
    fake = ctypes.c_void_p(0x10000)       # aligned non-null stand-in; never dereferenced
    odd = ctypes.c_void_p(0x10002)
    ptrs = [fake] * 11

    def fwd(p, H=256, I=128, E=4, Tp=640, pairs=18, M=5, variant=0):
        return L.rmoe_forward_f16_variant(*p, H, I, E, Tp, pairs, M, variant, None)

    assert fwd([None] + ptrs[1:]) == -1                   # null tokens
    assert fwd(ptrs, H=200) == -2                         # hidden not a multiple of 128
    assert fwd(ptrs, I=96) == -2
    assert fwd(ptrs, E=0) == -1
    assert fwd(ptrs, Tp=512) == -1                        # num_blocks_m*128 > Tp
    assert fwd(ptrs, pairs=-1) == -1
    assert fwd(ptrs, variant=7) == -1
    assert fwd([odd] + ptrs[1:]) == -3                    # misaligned fp16 tensor
    assert L.rmoe_gate_up_f16(*([fake] * 7), 256, 100, 4, 640, 18, 5, 0, None) == -2
    assert L.rmoe_gate_up_f16(*([fake] * 7), 256, 128, 4, 640, -1, 5, 0, None) == -1
    assert L.rmoe_down_f16(*([fake] * 8), 256, 128, 4, 640, -3, 5, 0, None) == -1
    assert L.rmoe_pack_f16(fake, fake, fake, fake, 3, 2, 12, fake, fake, 640, None) == -2
    assert L.rmoe_combine_f16(fake, fake, -1, 2, 16, fake, 640, None) == -1
    huge = 8 * ((1 << 30) + 1)  # rows beyond 2^30 16-byte chunks
    assert L.rmoe_pack_f16(fake, fake, fake, fake, 3, 2, huge, fake, fake, 640, None) == -2
    assert L.rmoe_combine_f16(fake, fake, 3, 2, huge, fake, 640, None) == -2
    assert L.rmoe_workspace_bytes(640, 128) == 640 * 128 * 2
    assert R.status_str(-5).startswith("tables violate")


def test_device_contract_argument_errors_without_gpu():
    """The device contract's argument checks also run before any HIP call."""
    L = R.lib()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10002)
    nb = ctypes.c_int32(-1)
    ws_ok = L.rmoe_contract_workspace_bytes(18, 4)
    # 18 pairs fit one 2048-pair chunk: (E + 1) int32 of per-chunk counts
    assert ws_ok == 1 * (4 + 1) * 4
    assert L.rmoe_contract_workspace_bytes(131072, 128) == 64 * 129 * 4
    assert L.rmoe_contract_workspace_bytes(10, 0) == 0
    assert L.rmoe_contract_workspace_bytes(10, 8193) == 0

    def dev(T=9, k=2, E=4, cap=5, ws=ws_ok, ids=fake, gs=fake, bad=fake, work=fake, nbp=ctypes.byref(nb)):
        return L.rmoe_build_contract_device(ids, T, k, E, gs, fake, fake, fake, cap, nbp, fake, fake,
                                            fake, bad, work, ws, None)

    assert dev(T=-1) == -1
    assert dev(E=0) == -1
    assert dev(E=8193, cap=10 ** 6) == -2                 # expert tables live in LDS
    assert dev(ids=None) == -1
    assert dev(gs=None) == -1
    assert dev(bad=None) == -1
    assert dev(work=None) == -1
    assert dev(nbp=None) == -1
    assert dev(cap=4) == -6                               # ceil(18/128) + 4 = 5 blocks needed
    assert dev(ws=ws_ok - 1) == -6                        # workspace too small
    assert dev(ids=odd) == -3
    assert nb.value == -1                                 # nothing written on an error


def test_router_argument_errors_without_gpu():
    L = R.lib()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)

    def rt(T=64, H=256, E=8, k=2, x=fake, ids=fake):
        return L.rmoe_router_f16(x, fake, T, H, E, k, ids, fake, None)

    assert rt(T=-1) == -1
    assert rt(E=0) == -1
    assert rt(k=9) == -1                                  # k > E
    assert rt(k=-1) == -1
    assert rt(E=257, k=2) == -2                           # E above the kernel's 256
    assert rt(E=64, k=33) == -2
    assert rt(H=96) == -2                                 # H not a multiple of 64
    assert rt(x=None) == -1
    assert rt(x=odd) == -3
    assert rt(T=0, x=None) == 0                           # nothing to do
    assert rt(k=0, ids=None) == 0


def test_fused_argument_errors_without_gpu():
    L = R.lib()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10002)

    def fz(H=256, I=128, E=4, Tp=640, pairs=18, M=5, sync=fake, x=fake, ho=0):
        return L.rmoe_forward_fused_f16(x, *([fake] * 10), sync, H, I, E, Tp, pairs, M, 0, ho, None)

    assert L.rmoe_fused_sync_words(5) == 16 + 5
    assert L.rmoe_fused_sync_words(-1) == 0
    assert fz(sync=None) == -1                            # the queue state is required
    assert fz(H=200) == -2
    assert fz(Tp=512) == -1
    assert fz(pairs=-1) == -1
    assert fz(x=odd) == -3
    assert fz(sync=ctypes.c_void_p(0x10002)) == -3        # int32 words
    assert fz(M=0, Tp=0, pairs=0) == 0                    # no blocks: nothing launched
    assert fz(ho=3) == -1                                 # unknown hand-over
    assert fz(ho=-1) == -1


def test_contract_sizes_and_variant_queries():
    """rmoe_contract_sizes is build_contract step 4 ("moe_dispatch_contract.py":
    m_blocks = ceil(pairs/128) + E) and agrees with the contract oracle's
    block count; rmoe_pick_variant is the one family choice of every entry."""
    for pairs, E in [(0, 1), (18, 4), (128, 8), (129, 8), (8192, 8), (49152, 64), (131072, 128)]:
        M, Tp = R.contract_sizes(pairs, E)
        assert M == -(-pairs // 128) + E and Tp == 128 * M
        ids = workloads.routing_from_counts([pairs // E] * (E - 1) + [pairs - (pairs // E) * (E - 1)])
        assert C.build_contract(ids.tolist(), E)["num_blocks_m"] == M
    L = R.lib()
    assert L.rmoe_contract_sizes(-1, 4, None, None) == -1
    assert L.rmoe_contract_sizes(10, 0, None, None) == -1
    assert L.rmoe_contract_sizes(2 ** 31, 4, None, None) == -1
    assert L.rmoe_contract_sizes(10, 4, None, None) == 0    # outputs are optional
    # streaming while the batch averages at most 96 rows per expert with at
    # most 4 experts, 56 with at most 8, 32 below 32 experts and 36 from 32
    # experts, tiling above
    assert R.pick_variant(128, 8) == "stream"               # decode workload
    assert R.pick_variant(288, 9) == "stream"
    assert R.pick_variant(289, 9) == "tile"
    assert R.pick_variant(448, 8) == "stream"
    assert R.pick_variant(449, 8) == "tile"
    assert R.pick_variant(384, 4) == "stream"
    assert R.pick_variant(385, 4) == "tile"
    assert R.pick_variant(992, 31) == "stream"
    assert R.pick_variant(993, 31) == "tile"
    assert R.pick_variant(1152, 32) == "stream"
    assert R.pick_variant(1153, 32) == "tile"
    assert R.pick_variant(8192, 8) == "tile"                # prefill workload
    assert R.pick_variant(8192, 8, "stream") == "stream"
    assert R.pick_variant(128, 8, "tile") == "tile"
    assert L.rmoe_pick_variant(7, 10, 4, -1) == -1
    assert L.rmoe_pick_variant(0, -1, 4, -1) == -1
    assert L.rmoe_pick_variant(0, 10, 0, -1) == -1
    assert L.rmoe_pick_variant(0, 10, 4, 11) == -1        # a group larger than the batch
    # the largest group weighs in when known: below 32 experts every expert
    # must fit one block
    assert R.pick_variant(128, 8, max_group_rows=23) == "stream"     # decode workload
    assert R.pick_variant(4096, 8, max_group_rows=100) == "tile"     # the average decides first
    assert R.pick_variant(384, 8, max_group_rows=128) == "stream"    # 8 experts, 48 rows, one block each
    assert R.pick_variant(384, 8, max_group_rows=129) == "tile"      # a group needs two blocks
    assert R.pick_variant(512, 16, max_group_rows=162) == "tile"     # E=16 Zipf, 32 rows per expert
    assert R.pick_variant(512, 16) == "stream"                       # largest group unknown
    # from 32 experts on the large groups' extra weight reads are a small share
    assert R.pick_variant(2048, 128, max_group_rows=120) == "stream"
    assert R.pick_variant(2048, 128, max_group_rows=242) == "stream"  # Zipf 1.2, 256 tokens
    assert R.pick_variant(2304, 64, max_group_rows=330) == "stream"   # Zipf 1.1, 384 tokens
    assert R.pick_variant(2305, 64, max_group_rows=54) == "tile"      # above 36 rows per expert
    assert R.pick_variant(5120, 128, max_group_rows=608) == "tile"    # Zipf 1.2, 640 tokens
    assert R.pick_variant(1024, 32, max_group_rows=208) == "stream"   # Zipf 1.2, 256 tokens
    assert R.pick_variant(2048, 128, "tile", max_group_rows=120) == "tile"
    # at most 32 experts, every group within one streaming pass: streaming
    # above the average threshold (largest group up to 64 rows; up to 96 at
    # an average of at most 80 rows with at most 8 experts, else 48)
    assert R.pick_variant(448, 8, max_group_rows=64) == "stream"     # 56 rows, one pass each
    assert R.pick_variant(512, 8, max_group_rows=75) == "stream"     # 64 rows, largest 75
    assert R.pick_variant(512, 8, max_group_rows=96) == "stream"
    assert R.pick_variant(512, 8, max_group_rows=97) == "tile"       # a group needs two passes
    assert R.pick_variant(640, 8, max_group_rows=94) == "stream"     # 80 rows, largest 94
    assert R.pick_variant(648, 8, max_group_rows=96) == "tile"       # 81 rows per expert
    assert R.pick_variant(1280, 32, max_group_rows=57) == "stream"   # E=32, 40 rows per expert
    assert R.pick_variant(1536, 32, max_group_rows=72) == "stream"   # E=32, 48 rows per expert
    assert R.pick_variant(1537, 32, max_group_rows=72) == "tile"
    assert R.pick_variant(720, 16, max_group_rows=64) == "stream"    # 45 rows, largest 64
    assert R.pick_variant(720, 16, max_group_rows=65) == "stream"    # 45 rows, largest 65 (<= 48 on average)
    assert R.pick_variant(784, 16, max_group_rows=65) == "tile"      # 49 rows, largest 65
    assert R.pick_variant(576, 9, max_group_rows=65) == "tile"       # 64 rows with 9 experts
    assert R.pick_variant(576, 9) == "tile"                          # largest group unknown
    assert R.pick_variant(2560, 33, max_group_rows=64) == "tile"     # more than 32 experts


def test_validate_device_argument_errors_without_gpu():
    L = R.lib()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10002)

    def vd(E=4, M=5, Tp=640, pairs=18, viol=fake, gs=fake):
        return L.rmoe_validate_contract_device(gs, fake, fake, fake, E, M, Tp, pairs, viol, None)

    assert vd(viol=None) == -1
    assert vd(gs=None) == -1
    assert vd(E=0) == -1
    assert vd(gs=odd) == -3
    assert vd(M=6) == -5                                  # not ceil(18/128) + 4
    assert vd(Tp=512) == -5                               # 5 blocks do not fit 512 rows
    assert vd(pairs=-1) == -1


def test_binding_holds_no_contract_arithmetic():
    """The Python binding only marshals: block counts, padded sizes and the
    family choice come from the library (rmoe_contract_sizes,
    rmoe_pick_variant), so no formula of the contract is written there."""
    import ast
    src = open(os.path.join(ROOT, "mixture_experts_routed_grouped_amd", "__init__.py")).read()
    tree = ast.parse(src)
    for node in ast.walk(tree):
        # a number 128 (the block size) or 32 (the streaming threshold)
        # anywhere in the binding would be contract or policy arithmetic
        if isinstance(node, ast.Constant) and node.value in (128, 32):
            raise AssertionError(f"binding line {node.lineno}: constant {node.value}")
        if isinstance(node, ast.Name) and "BLOCK_M" == node.id.upper():
            raise AssertionError(f"binding line {node.lineno}: {node.id}")
    for name in ("bench.py", "__graft_entry__.py"):
        text = open(os.path.join(ROOT, name)).read()
        assert "32 * E" not in text and "-(-" not in text, name


def test_noalloc_contract_limits_without_gpu():
    """The allocation-free contract build checks its batch against the static
    scratch before any HIP call."""
    L = R.lib()
    fake = ctypes.c_void_p(0x10000)
    nb = ctypes.c_int32(-1)
    words = L.rmoe_contract_noalloc_max_words()
    assert words == 1 << 18

    def na(T, k, E, cap=10 ** 7):
        return L.rmoe_build_contract_device_noalloc(fake, T, k, E, fake, fake, fake, fake, cap,
                                                    ctypes.byref(nb), fake, fake, fake, fake, None)

    # E = 8192: 49 chunks of 2048 pairs need 49 * 8193 words > 2^18
    assert na(100000, 1, 8192) == -7
    assert na(-1, 1, 4) == -1
    assert na(10, 1, 8193) == -2
    assert na(300, 1, 4, cap=4) == -6
    assert nb.value == -1
    assert R.status_str(-7).startswith("batch exceeds")
