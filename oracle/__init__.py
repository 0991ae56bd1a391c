"""Plain fp64 CPU oracle of one DSpark draft-and-verify round.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
anything in this package: only the tests, the smoke check of the entry script
and the CPU-baseline leg of the benchmark do.  The oracle shares no code with
the HIP path (no kernels, headers, helpers or constant tables); the two meet
only through the seeded input generators, which hold none of the method's
arithmetic.

Sources (the pages):
  * "Les mathématiques derrière l'accélération ..." (seventnews.com), section
    "La garantie de l'échantillonnage par rejet": the acceptance rule
    min(1, p/q), stop at the first rejection, resample from the residual;
    section "Rendement attendu et formule d'accélération": expected tokens per
    verification pass (1 - a^(g+1)) / (1 - a).
  * "DSpark, la bozza che sa quando fermarsi" (paithon.it), section "Un po' di
    autoregressione basta": the draft distribution p_k (eq. p_k) with the Markov
    head B = W1 W2 of rank 256; section "Verificare meglio, non di più": the
    analytic acceptance c*_k, prefix survival a_j = prod c_i, Theta = tau SPS(B)
    and the greedy early-stop admission.
  * "DeepSeek发布DSpark" (learnblockchain.cn), section "DSpark 是什么？": the bonus
    token after a fully accepted prefix.

Modules:
  philox   -- Philox4x32-10 counter-based generator and the uniform/Gumbel maps
  sampler  -- the three-level Gumbel-max categorical sampler
  dspark   -- draft round, verify, scheduler, and probability helpers
  ref      -- ctypes binding of the C oracle (dspark_ref.c: the ref_ entry
              points, the same round as plain fp64 loops with OpenMP over
              requests; compiled by build.py), pinned against dspark
"""

from . import philox, sampler, dspark  # noqa: F401
