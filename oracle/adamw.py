"""Oracle of the optimizer step applied to the LoRA adapters.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages introduce paged optimizers -- optimizer state that is moved to CPU
memory during memory spikes ("QLoRA: Efficient Fine-Tuning of Quantized
Language Models" (mbrenndoerfer.com), section "Paged Optimizers"; "QLoRA:
Efficient Finetuning of Quantized LLMs", Introduction, contribution (3)) --
but name no update rule. READING: Adam with bias-corrected moments and
decoupled weight decay (AdamW), state and master weights in float32, the
gradient in bf16 as the backward produces it. Where the state lives does not
change the arithmetic, so one oracle serves every placement.
"""

import numpy as np


def adamw_step(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay):
    """One AdamW step in float64. Returns (p_new, m_new, v_new).

    m <- beta1 m + (1 - beta1) g
    v <- beta2 v + (1 - beta2) g^2
    p <- p - lr (weight_decay p + m_hat / (sqrt(v_hat) + eps)),
         m_hat = m / (1 - beta1^step), v_hat = v / (1 - beta2^step)
    ``step`` counts from 1. Weight decay uses the parameter before the update.
    """
    if step < 1:
        raise ValueError("step counts from 1")
    p, g, m, v = (np.asarray(t, dtype=np.float64) for t in (p, g, m, v))
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    p_new = p - lr * (weight_decay * p + m_hat / (np.sqrt(v_hat) + eps))
    return p_new, m_new, v_new
