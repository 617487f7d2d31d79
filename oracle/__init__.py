"""CPU oracle for the CSA / HCA compressed-attention hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, fp64 numpy (plus
pure-Python for tiny sizes) restatement of what the method computes.  Only the
test suite, the package-level smoke check and the benchmark's CPU-baseline leg
may import it.  The GPU library never imports, links or calls anything here,
and nothing here imports the GPU library: the two share no code.

Sources.  The method is described on five web pages about DeepSeek-V4; each
function cites the page (by site and title) and the section it follows.  The
pages name the compressor and the indexer without defining them; the two
definitions used here (a softmax-weighted pool with one scalar logit per token,
and the indexer score sum_h w_h * ReLU(q_h . k_e) on MXFP4 operands) are fixed
by the project, not the pages, and are marked "parity unpinned by the pages"
where they are used: only the arithmetic that follows from them is pinned.

Modules
  formats    number formats: bf16, OCP E4M3FN (fp8), E2M1 / MXFP4
  compress   softmax-pool KV compression (CSA block m, HCA block m')
  indexer    lightning-indexer scores
  topk       top-k selection with the lower-index tie rule
  attention  CSA sparse attention and HCA dense attention (+ window branch)
  brute      pure-Python loop versions of all of the above, for tiny inputs
"""
