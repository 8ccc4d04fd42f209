"""fp64 CPU oracle for the streaming semi-Markov CRF — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding in ``semi_markov_crf_amd``) never imports, calls or links
anything here, and nothing here imports the product path.  The two share no
code: only the seeded generators in ``workloads.py`` (random draws, no method
arithmetic) feed both.

The oracle is the plain definition written out in NumPy float64: it
materialises the dense edge-potential tensor (in tiles of segment start
positions) and runs the textbook semi-CRF forward, backward, posterior and
max-plus recursions over it.  See ``oracle/semicrf.py`` for the definitions,
their citations and the readings taken where the pages are silent.
"""

from .semicrf import (  # noqa: F401
    centered_prefix,
    edge_potentials,
    forward,
    backward,
    posteriors,
    viterbi,
    segmentation_score,
    sequence,
    batch,
    gold_features,
    nll_sequence,
    nll_batch,
)
