"""CPU oracle for the TwELL sparse ReGLU feed-forward forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package never imports the product path: the two share no
code.  Inputs come from the seeded generators in ``workloads/``.

What the oracle computes, and which passage each part follows:

* ``ffn``: the plain dense FFN y = (ReLU(x W_g^T + beta) * (x W_u^T)) W_d in
  float64.  Exploiting the post-ReLU zeros is an exact reformulation (zero
  activations contribute nothing), so the dense formula *is* the result the
  sparse path must reach: gist.science "Sparser, Faster, Lighter Transformer
  Language Models", Resumen Técnico §2.B (inference kernel: up and down
  projections driven by the gate activations) and the edge.aivizor.me news
  post on TwELL (second paragraph: the architecture is unchanged, only work
  for neurons that did not fire is skipped).  ReLU in place of SiLU: q2bstudio
  post on TwELL (fourth paragraph) and the same Resumen Técnico §5.
* ``twell``: the TwELL (tile-wise ELLPACK) packer / unpacker and the hybrid
  dense-backup rows for overflowing rows: Resumen Técnico §2.A (columns cut
  into tiles, non-zeros packed per tile; overflow rows go to a dense backup
  matrix) and the q2bstudio post (third paragraph: compact ELL plus dense
  backup for rows with many non-zeros).  The pages fix no field layout; the
  layout used here is the one declared in ``include/twell.h``.
* ``hybrid``: the hybrid training format (compact ELL rows plus a dense
  backup for rows with many non-zeros) and its conversion from TwELL:
  Resumen Técnico §2.A (hybrid format for training) and §2.B (training
  kernels: TwELL to hybrid conversion).
* ``penalty``: the L1 activation penalty ||h||_1 and its gradient, from
  TwELL: Resumen Técnico §2.B (training strategy: L1 regularisation of the ReLU activations)
  and §4 (coefficient 2e-5).
* ``backward``: the gradients of the layer (dx, dW_g, dW_u, dW_d) with the
  L1 penalty, from the stored activations in hybrid form: Resumen Técnico
  §2.A (hybrid activations kept for back-propagation) and §2.B (training
  kernels: hybrid-dense and dense-hybrid products, sparse transpose).
* ``numerics``: exact decoding of the storage dtypes to float64 and
  round-to-nearest-even encoding to bf16.

Every function here is pinned by ``-m "not gpu"`` tests against exact
rational arithmetic, hand-worked examples, closed forms, invariants, and for
the backward pass automatic differentiation and finite differences.
"""

from .numerics import decode, round_to_bf16, round_to_storage, storage_zero  # noqa: F401
from .ffn import ffn, ffn_from_h, gate_pre, rel_l2, row_rel_l2  # noqa: F401
from .twell import (  # noqa: F401
    Packed,
    active,
    pack,
    pack_loop,
    relu_storage,
    sparse_ffn,
    tile_major,
    unpack,
)
