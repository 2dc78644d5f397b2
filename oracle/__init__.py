"""CPU oracle for confidence-scheduled speculative decoding.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
statement of what the GPU path computes.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
it.  The product path (``draft_verification_amd``) never imports, links or
executes anything here, and nothing here imports the product path.

Arithmetic is float64 NumPy unless a step's definition fixes another precision
(the survival products are fp32 by definition, the drafted logits are rounded
to bf16 by definition).  Loops are plain Python so that each step can be read
against the pages by eye.

Sources (cited by page title and section):
  * "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
    Generation" (paper summary page): section "2.1 confidence head",
    "2.2 hardware-aware prefix scheduler", Figure 1, "challenge 2: async
    scheduling and ZOS", "innovation one" (Markov and RNN sequential heads).
  * speculative-decoding history page: "1.1 mechanism" (draft, parallel verify,
    rejection sampling, losslessness), DSpark "move one" (Markov head) and
    "move two / move three" (survival products, greedy scheduler).
  * LightSpec article: the two-stage budget planner (verify budget, then draft
    budget), runtime statistics kept as EMAs with interpolation across draft
    lengths, runtime cost tables; reserving token slots at the maximum draft
    length.

Parity status per function is stated in each module header.
"""

from . import rng, schedule, verify, markov, bf16, lightspec, rnn  # noqa: F401
