"""CPU oracle for the dequant-fused projection matmul.  TEST INFRASTRUCTURE.

    dst[j, i] = sum_c deq(W)[i, c] * x[j, c]      (0 <= i < m, 0 <= j < n)

(cera `examples/wgpu_gemm_bench.rs`, the Shape doc comment: one benchmarked
matmul is dst[n, m] = src0[m, k] * src1[n, k]; dst is column-major with
y_stride = m, i.e. dst[j*m + i].)

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path: it decodes every block format
from its definition, in float64, and contracts with a plain f64 matmul.

Modules
  formats  vectorized numpy block decoders (exact in f64) + element codecs
  scalar   a literal per-element pure-Python decoder for tiny inputs
  ref      the f64 reference GEMM, MoE gate/up, SwiGLU/clamp activation and
           down projection (f32 or Q8_1 activations), and the tolerance scale S

Every decoder is pinned in ``tests/test_oracle_*.py`` against hand-built
blocks, library routines (numpy float16, torch float8/float4 dtypes),
test-only encoders and brute force.  The one part with no pin is the meaning
of the bit layouts on real checkpoints ("parity unpinned": no GGUF or NVFP4
file is available to compare against).
"""

from .formats import (  # noqa: F401
    QTYPES,
    qtype_id,
    block_elems,
    block_bytes,
    row_bytes,
    f16_bits_to_f64,
    e4m3_bits_to_f64,
    e2m1_bits_to_f64,
    decode,
)
from .ref import gemm_ref, gemm_ref_rows, gemm_value, moe_ref, tolerance_check  # noqa: F401
