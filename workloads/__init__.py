"""Seeded synthetic inputs for exact tensor-network contraction.

This package only *describes and fills* inputs: networks (mode labels,
extents, leaf mode lists, the output order), leaf data drawn from
``numpy.random.default_rng(seed)``, and contraction trees chosen by a
deterministic greedy rule.  It performs none of the contraction arithmetic,
so both the CPU oracle and the GPU path can take their inputs from it.

Workload families (stand-ins for the circuits and lattices named on the
source page "Parallelizing Large-Scale Tensor Network Contraction on Multiple
GPUs", sections 2.1-2.3, whose definitions are not given there):

* random brickwork circuits with Haar-random two-qubit unitaries,
* random 2-D grid circuits with fSim-form couplers,
* an 8x8 square-lattice (PEPS-style) partition-function network,
* isolated pairwise contractions (the GEMM sweep),
* honeycomb-lattice and graph Ising partition functions (``hexagonal``),
* surface-code decoding (coset-weight) networks (``qec``),
* small random networks for property tests.
"""

from .network import Network, Tree
from . import circuits, lattice, sweep, trees, randnet

__all__ = ["Network", "Tree", "circuits", "lattice", "sweep", "trees", "randnet"]
