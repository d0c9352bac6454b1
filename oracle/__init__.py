"""CPU oracle for the packed NR-MMDiT block and its rectified-flow wrapper.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test-suite, the smoke check of the entry module and the CPU-baseline
leg of the benchmark may import or call it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constant generators).

Every function is the plain definition of what the method computes, written
sample by sample in float64 with no blocking or fusion, so that a reader can
check it against the pages by eye.  The pages the citations refer to:

* "hyper.ai 2607.19064" -- the hyper.ai summary page of arXiv 2607.19064,
  sections 方法 (method) and 实验 (experiments).
* "blog close-reading" -- the Obsidian-blog close reading of the paper
  "Mage-Flow: An Efficient Native-Resolution Foundation Model for Image
  Generation and Editing", sections 2.2 (mechanism) and 5 (concepts).

Where the pages leave a step open, the reading taken is named in the
function's docstring as R<n>; the full list of readings lives with the
design notes of the repository.

Modules:
  pack   -- native-resolution packing: plan, offsets, segment and position ids
  block  -- timestep conditioning, adaLN, RMSNorm, QK-norm, 3-axis RoPE,
            joint attention, the dual-stream block and the final layer
  flow   -- rectified-flow noising, loss, CFG combine and Euler sampling

Parity status: pack, flow, RMSNorm, RoPE, attention and GELU are pinned by
closed forms, invariants, library routines and brute force (tests marked
"not gpu").  The composition of the whole block (order of sub-steps, adaLN
chunk order, final layer) follows readings of the pages; beyond the
adaLN-zero identity, packed-CFG equivalence and the torch.nn.functional
composition check it is "parity unpinned".
"""

from . import pack, block, flow  # noqa: F401
