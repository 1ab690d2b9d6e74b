"""fp64 CPU oracle of the CCA / CCGQA forward and backward pass -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The GPU library never
calls it and shares no code with it.

Modules
-------
``cca``    vectorised NumPy oracle (prefill, sampled-row prefill, decode step,
           multi-token decode step)
``brute``  scalar pure-Python twin for tiny inputs, written separately
           from the same readings, used to pin ``cca``
``backward``  the derivative of every step of ``cca`` (chain rule, fp64) and
           the whole prefill backward pass

Every step cites the passage of the pages that defines it.  Page tags:

* [ABS]     mlsanity.com, "Compressed Convolutional Attention: Efficient
            Attention in a Compressed Latent Space", section "Abstract (arXiv)"
* [GS-EN]   gist.science, English explainer of the same paper; sections
            "1. Problem Statement", "2. Methodology", "3. Key Contributions"
* [GS-DE]   gist.science, German explainer of the same paper; section
            "2. Methodik"
* [EDG]     blogs.edgentiq.com, "Boosting Transformer Efficiency with
            Compressed Convolutional Attention"; sections "How Compressed
            Convolutional Attention Works" and "Introducing CCGQA"

Where the pages leave a step open, the oracle takes one stated reading; the
steps that rest on such a reading are marked "parity unpinned" below and in
the design notes: the channel convolution's form (per-head taps sliding
along the channel index, or the grouped switch: dense d x d weights per lag
and head), the exact q-k-mean formula, the temperature value,
the RoPE pair convention, and which half of the value heads is shifted.
"""

from .cca import (  # noqa: F401
    Readings,
    DEFAULT_READINGS,
    down_project,
    seq_conv,
    chan_conv,
    chan_conv_grouped,
    conv_window_rows,
    qk_mean,
    value_shift,
    l2_normalize,
    rope,
    rope_angles,
    causal_attention,
    up_project,
    latents,
    prefill,
    prefill_state,
    decode_step,
    decode_multi,
)
