"""CPU oracle for the quantized Mamba2 mixer layer of the FastMamba method.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  The product path
(the HIP library ``libfm.so`` and its Python binding) never imports, calls or
links anything here, and nothing here imports the product's kernels, headers
or binding: the two sides share no code.  The only shared module is the
seeded input generator ``quantized_state_space_fwht_amd.synth``, which draws
numbers and holds no step of the method.

Plain numpy, slow and direct.  Floating point is float32 where the method
turns a float into an integer code (the decision is taken in the precision the
kernels use, IEEE float32 with no fused multiply-add); integer and fixed-point
stages are exact int64 arithmetic.  Every function cites the passage it
follows, using these short names for the pages:

[FM]   "FastMamba: A High-Speed and Efficient Mamba Accelerator on FPGA with
       Accurate Quantization" (arXiv 2505.18975), the pith.science review page:
       "What carries the argument", the referee report (summary; major comment
       on Sections III-A / IV-B about Algorithm 1 and Fig. 6; minor comment on
       Section III-B.2 about Eq. (5)), the abstract, and the figure captions
       (Fig. 2 Mamba2 block flow, Fig. 3 activation distributions).
[FMV]  the same paper's verdict record on pith.science: the skeptic critique
       (static calibrated scale, multiply+shift) and the supporting citations
       ([14] zero-order hold, [15] shift-based exponential for e^dt,
       [16] SoftPlus symmetry).
[MPTQ] "Mamba-PTQ: Outlier Channels in Recurrent Large Language Models",
       abstract (outlier channels in Mamba activations).

Where the pages leave a step open the docstring says "reading:" and states the
choice.

Pinning: tests/test_oracle_pins.py checks every function here against
mathematics the pages fix or a library routine (see each test's docstring).
"""
from .fixedpoint import (I32_MAX, I32_MIN, PMAX, PMIN, f32_to_i32_sat, pot_f32, pot_q16, rshr,
                         sat8, sat32)
from .hadamard import fwht256_f32, hadamard_quant, hadamard_scale, quantize_codes
from .linear import quantize_weight, w8a8_gemm
from .nau import (EXP2_TABLE_Q30, LOG2E_Q30, exp2_q16, exp_q16, silu_q16, softplus_q16)
from .conv import conv1d_pot, conv_weight_prep, silu_requant, xbc_pot_quant
from .scan import (dt_dA, narrow_state, pack_state, ssm_scan_pot, ssm_scan_real, state_shift_for,
                   unpack_state, widen_state)
from .gate_norm import gate, gate_norm_quant, rmsnorm_fixed_order
from .layer import (QParams, Stats, calibrate_stack, layer_decode, layer_prefill, prepare_layer,
                    qparams_from_stats, stack_decode, stack_prefill)
from . import outliers, quant_stats
