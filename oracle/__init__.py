"""CPU oracle for the forward pass of one DeepSeek-V3 MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never calls it, and the
oracle never imports the product package: the two share no code.

The oracle is plain numpy in float64.  It emulates the fixed rounding points of
the method (BF16 inputs, FP8 E4M3 codes with FP32 scales, FP32 GEMM outputs,
BF16 expert outputs and layer output) and otherwise computes exactly.  Sources
are the five pages about the DeepSeek-V3 technical report; citations name the
page title and the section on it.

Modules
-------
fp8      E4M3 and BF16 rounding written from the bit-field definitions.
quant    1x128 activation tiles and 128x128 weight blocks, online amax scaling.
route    sigmoid affinity, selection-only bias, group-limited top-k, gates.
permute  stable grouping of (token, expert) assignments by expert.
gemm     blocked FP8 GEMM with one FP32-visible partial sum per 128-wide K block.
layer    SwiGLU experts, shared expert, combine, and the whole layer.

Pins (what each function is checked against, in ``tests/test_oracle_*.py``)
--------------------------------------------------------------------------
fp8.e4m3_*      the format table on "DeepSeek-V3: the recipe, and the interconnect
                that shaped it" (FP8 section: max 448, min normal 1.562e-2, 8 steps
                per octave); exhaustive decode of all 256 codes; torch's
                float8_e4m3fn conversion (an independent library) on every code
                midpoint and its FP32 neighbours; RNE tie cases by hand.
fp8.bf16_*      torch's bfloat16 conversion on random and tie inputs.
quant.*         exact round trip of values already on the E4M3 grid; the quiet-value
                error statistic printed on the same page (block 128: 0.026348) as a
                loose statistical pin; the 4096x7168 byte count (30.28 MB); the FP32
                rule scale = fl32(amax/448), code = E4M3(fl32(x/scale)) against exact
                rational arithmetic on a non-power-of-two scale, on values where a
                reciprocal multiply gives another code, and on values where
                fl32(x/scale) lands on an E4M3 midpoint that x/scale does not
                (tests/test_oracle_quant_rule.py); the power-of-two rule against hand
                values and an enumeration of exponents.
route.route     the two worked examples of the book's chapter 7 ("A toy mixture")
                and chapter 8 ("A selection-versus-weighting example"); brute-force
                enumeration of group subsets and expert subsets on tiny inputs;
                invariants (k distinct ids, at most M groups, gates sum to 1,
                bias-independence of the gates given the set).
permute.*       brute-force Python loop; bijection; combine(permute(x)) round trip.
gemm.blocked    dense float64 GEMM of the dequantised operands (a textbook identity);
                K = 128 reduces to a single scaled dot product.
layer.*         SwiGLU closed form; k = E dense special case; route_scale = 0 gives
                the shared expert alone; sampled-token evaluation equals the
                full-batch evaluation.

Every function above has at least one pin that does not restate its own
formula.  What no pin reaches: the whole-layer output at the V3 shape (no page
prints one); it rests on the pins of its parts and on the k = E dense case.
"""

from . import fp8, quant, route, permute, gemm, layer  # noqa: F401
