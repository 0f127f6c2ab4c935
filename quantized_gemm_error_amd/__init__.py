"""MI355X-native compensated 4-bit linear layer (libspear) and its Python binding."""

from .spear import (  # noqa: F401
    SPEAR_BF16,
    SPEAR_F16,
    SpearError,
    SpearLayer,
    act_to_device,
    layer_to_device,
    load_library,
    new_workspace,
    spear_get_decode_max_m,
    spear_last_error,
    spear_linear,
    spear_linear_decode,
    spear_linear_prefill,
    spear_pack_int4,
    spear_select_chunk,
    spear_set_decode_max_m,
    spear_status_string,
    spear_version,
    spear_workspace_bytes,
    spear_workspace_flags,
)
