"""fp64 CPU oracle of the AdamW companion step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library and
imports nothing from it.

Sources.  The pages' optimizer takes a separate AdamW learning rate
(``adamw_lr=1e-3``) next to Muon's ``lr`` and ``ns_steps``, for the parameters
that its predicate does not route to Muon -- embeddings, norms, heads (DMuon
project documentation, quick-start snippet and the VLA/VLM paragraph).  The
pages give no other AdamW hyperparameter.  The reading taken here is the usual
decoupled-weight-decay Adam with bias correction and the defaults of the common
deep-learning frameworks: betas (0.9, 0.999), eps 1e-8, weight decay 0.01.

Per element, at step t >= 1, in fp64 (bf16 and fp32 inputs embed exactly):

1. decoupled decay:  p <- p (1 - lr wd)
2. first moment:     m <- beta1 m + (1 - beta1) g
3. second moment:    v <- beta2 v + (1 - beta2) g^2
4. bias correction:  m_hat = m / (1 - beta1^t),  v_hat = v / (1 - beta2^t)
5. step:             p <- p - lr m_hat / (sqrt(v_hat) + eps)

Pins (tests/test_adamw_oracle.py): the first step's closed form
-lr g / (|g| + eps), a constant gradient's closed form at any t, zero gradient
(decay only), and several steps against torch.optim.AdamW run on the CPU in
float64 (an independent implementation of the same update).
"""

from __future__ import annotations

import numpy as np

ADAMW_DEFAULTS = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def adamw_step(p, g, m, v, step, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
    """One AdamW step on one tensor; returns (p', m', v') in fp64.

    ``step`` is the 1-based count of steps taken including this one.
    """
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
