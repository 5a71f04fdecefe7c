"""Plain CPU oracle of one Medusa tree-verification round.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package.  The HIP library never
routes through it and shares no code, header, table or helper with it.

Every function is a slow, direct transcription of what the pages define,
computed in IEEE binary64 unless the operation is integer-only:

* ``tree``       -- rank-path tree compilation and greedy budgeted growth
* ``attention``  -- tree attention as one ordinary causal attention per
                    root-to-node path, plus the staged K/V rows
* ``accept``     -- greedy longest-prefix acceptance (two independent ways)
* ``typical``    -- fast typical acceptance
* ``compact``    -- winning-path K/V compaction with a snapshot
* ``heads``      -- the Medusa head step and the ranked candidate pool

Pages cited (by title and section):

[M7.2]  "M7.2 - Medusa: Multi-Head Candidates, Tree Attention, and Verification"
[Chai]  "Medusa 完全拆解：多头树式候选如何用一次验证解码多个 Token"
[PartII] "Medusa Part II: Candidate Trees, Verification, and Acceptance"
[Math]  "Medusa — Multi-Head Speculative Decoding Math"
"""

from . import tree, attention, accept, compact, typical, heads  # noqa: F401
