"""Oracle for the routed fused-MoE expert FFN -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously correct CPU definition that the
HIP path is checked against.  It shares no code with the HIP path and does
not import it.  Only the tests, the smoke check and the benchmark's CPU
baseline may import anything from here; the product path never does.

Modules
-------
contract : host-side dispatch contract (group tables, stable order, packing)
           and its invariants, from the tutorial page "moe_dispatch_contract.py"
           (function build_contract and its three self-checks).
ref      : ctypes front end of ``moe_ref.c``: the per-row fused expert FFN in
           plain C with fp32 accumulation and fp16 rounding of the hidden
           workspace and the output, from "Fused MoE GEMM 提交说明",
           section 算子来源 (computation semantics) and 完整算子代码 (dtypes).
brute    : per-(token, expert) dense loop in float64 numpy that uses no
           contract table at all; for tiny inputs.
combine  : the k-way combine of the expert outputs back into token order
           (fp32 sum in slot order, one fp16 rounding).
router   : router logits, softmax over the experts and top-k in float64,
           from "MetaX-TileLang工具链", section 2.4.
build    : compiles ``moe_ref.c`` with gcc into ``oracle/_build``.
"""
