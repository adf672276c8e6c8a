"""CPU oracle for block-sparse video-DiT attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything here: only the tests, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg use it.  It shares no code with the HIP library; the
two meet only through the seeded generators in ``workloads.py``.

Each module is a plain, slow, obviously correct restatement of what the pages
define, in float64 unless the definition fixes another precision:

* ``crm``          -- the packed row-mask format and its forward iterator
                      (ScalingAttention, section 4.3.2 and Appendix E, Alg. 2).
* ``attention``    -- softmax(scale * Q K^T + M) V over kept blocks, M in {0,-inf}
                      (ScalingAttention, section 4.3.2; density definition in
                      Figure 1 and section 5.1).
* ``stripes``      -- PSA stripe tuples expanded to a block mask (PSA page,
                      Figure 3 and Appendix Tables 7-9).
* ``block_scores`` -- mean-pooled block proxy scores (SCOPE abstract; block
                      aggregation as in ScalingAttention Eq. 1).
* ``topp``         -- hybrid top-p / top-k-minimum block selection (Competition
                      Domains abstract, SCOPE abstract, ScalingAttention Alg. 1
                      cumulative-mass cut-off) as a fixed float32 procedure.
* ``hilbert``      -- 3D Hilbert token order (DFSAttn abstract), Skilling's
                      transpose construction.
* ``threshold``    -- mask instantiation M = I(T <= p*) from a threshold map
                      (ScalingAttention section 4.1.2, Eq. 2; Algorithm 1).
* ``fidelity``     -- Hellinger distance / Fidelity Score between dense and
                      sparse attention rows (ScalingAttention Eqs. 3-4,
                      section 4.2.3 stratified rows).
* ``resize``       -- resolution scaling of region / threshold maps
                      (ScalingAttention section 4.3.1, Eq. 7).
"""
