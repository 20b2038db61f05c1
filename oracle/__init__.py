"""CPU oracle for the W4A4G4 triple-branch linear (test infrastructure).

This package is test infrastructure, not part of the product: only the
tests, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it.  It shares no code with the GPU library.

It follows FourTune ("FourTune: Towards Fully 4-Bit Efficient Post-Training
for Diffusion Models"):

* quantizer Q(.) in 16x16 blocks, E2M1 codes plus one scale per block
  (section 3.1, Eq. 2 and the definition of Q(.) after it; section 3.2,
  block-wise quantization; section 4.3, "Impact of Quantization
  Granularity"), with scale = block amax / 6 and round-to-nearest-even;
* forward Y = GEMM_4bit(Q(X), Q(R)) + X L_stab + X (A B) (section 3.1, Eq. 2);
* backward dX = GEMM_4bit(Q(G), Q(R)^T) + G L_stab^T + G (A B)^T (section
  3.2, Eq. 3) and dB = (X A)^T G, dA = X^T (G B^T) (section 3.2);
* the offline split W ~= R + L1 L2 (section 3.1, Eq. 1) is checked, not
  produced, here;
* the other quantization granularities of section 4.3 ("Impact of
  Quantization Granularity", Table 5): 1 x g groups along rows (g = 16, and
  g = 32, the group the gfx950 block-scaled instruction takes), and the
  backward's re-quantization of the transposed weight that group scales
  force (section 3.2).

Everything is evaluated in fp64 on exactly dequantized values.  Every
function is pinned by a ``-m "not gpu"`` test against brute force, exact
rational arithmetic, closed forms or special cases; none is "parity
unpinned".
"""
from .ft_oracle import *  # noqa: F401,F403
from .ft_oracle import __all__  # noqa: F401
