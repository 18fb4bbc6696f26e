"""CPU oracle for kernelized linear attention (test infrastructure only).

Only tests, the smoke check and the bench's CPU-baseline leg may import this
package. It shares no code with the HIP library or its binding.
"""

from .linattn_oracle import (  # noqa: F401
    EPS,
    FMAPS,
    attention,
    attention_backward,
    attention_via_state,
    chunked,
    cumsum_form,
    decode_step,
    feature_dim,
    feature_map,
    feature_map_vjp,
    final_state,
    gated_attention,
    gated_chunked,
    gated_decode_step,
    gated_final_state,
    gated_recurrent,
    phi_elu1,
    phi_identity,
    phi_performer,
    phi_poly2,
    recurrent,
    recurrent_backward,
)
