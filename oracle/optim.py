"""The optimizer step of the adapter parameters (CPU oracle, fp64).

Test infrastructure only (see the package docstring).

What the pages say: QLoRA trains only the adapters with a paged optimizer
(apxml.com "量化 LoRA (QLoRA) 与 4 位训练", the paged-optimizer paragraph:
optimizer state is moved between GPU memory and system CPU memory when GPU
memory runs short; ai-reference-codex "QLoRA 与 PEFT 全家", §3.3: the state is
moved out to host memory while memory is tight and moved back afterwards, the
configuration being paged_adamw_32bit, and §4: that optimizer with learning
rate 2e-4; aivaro.ru "Как работает QLoRA", §6: Adam keeps two values per
trained parameter, the first and second moments, which are paged out to the
CPU and back).

The pages give no update formula. Reading: AdamW as published (Adam, Kingma
and Ba 2015, Algorithm 1, with its bias corrections; the weight decay
decoupled from the gradient as in Loshchilov and Hutter 2019, AdamW), with
32-bit state: the two moments and the parameter are fp32 between steps. One
step t >= 1 on parameter p with gradient g:

    m  = b1 m + (1 - b1) g
    v  = b2 v + (1 - b2) g^2
    m^ = m / (1 - b1^t),   v^ = v / (1 - b2^t)
    p  = p - lr (m^ / (sqrt(v^) + eps) + wd p)

Where the state lives (device or host memory) does not change the values:
paging moves the state, the step is the same.
"""

import numpy as np


def adamw_step(p, g, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """One AdamW step in fp64 on 1-d arrays (copies; the inputs are not
    modified). Returns (p, m, v) after the step; ``step`` is the step
    number t of this update, counted from 1."""
    if step < 1:
        raise ValueError("the step number counts from 1")
    p = np.asarray(p, dtype=np.float64).copy()
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64).copy()
    v = np.asarray(v, dtype=np.float64).copy()
    b1, b2 = float(beta1), float(beta2)
    # first and second moment estimates
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * (g * g)
    # bias-corrected estimates
    m_hat = m / (1.0 - b1**step)
    v_hat = v / (1.0 - b2**step)
    # decoupled weight decay on the parameter before the step
    p = p - float(lr) * (m_hat / (np.sqrt(v_hat) + float(eps)) + float(weight_decay) * p)
    return p, m, v
