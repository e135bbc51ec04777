"""CPU oracle for the Leech-lattice dequantize-plus-matvec path.

THIS PACKAGE IS TEST INFRASTRUCTURE.  It is a plain, slow, obviously correct
reference written from the pages (the arXiv paper "Unfolding the Leech Lattice:
Fused Multi-Shell Decoding and VRAM Layouts for 2-Bit LLM Weights", the Tetra
summary, the model card "Qwen3-8B - 2-bit BPDQ (packed)" and the blog post
"Qwen3.8-27B on a 12 GB card"), in float64 and exact integer arithmetic.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and nothing here imports the product
path.

Modules
-------
golay   the extended binary Golay code G24 (classical construction).
leech   Leech-lattice membership, shells, coordinate-permutation classes and
        their exact point counts, the theta-series closed form.
gemv    f64 reconstruction of W for every arm (Leech, BPDQ, bitshift trellis,
        dense fp16) and the f64 matvec with its per-row error bound.
layout  the expected logical planes of a Leech block and an independent
        unpacker of the packed blob the expander writes.
rotate  the activation rotation (H kron Q)(S x) with its error bound.
index   the 47-bit rank / unrank of the m <= 12 ball, the 48-bit word and
        shape-gain dequantisation.

Parity status: every function is pinned by a CPU test against a value the
pages print, a classical closed form, or brute force; the exceptions are
listed as "parity unpinned" in the docstrings that carry them.
"""
