"""Seeded synthetic inputs shared by the oracle checks and the GPU path (no layer arithmetic)."""
from .configs import (ALL, DECODE, FWD_BF16, FWD_MXFP8, SHARE_BF16, SHARE_MXFP8, SKEW_BWD,
                      TINY_F32, LayerConfig, ShareConfig)
from .inputs import (LayerInputs, ShareInputs, bits16, host_f32, make_layer, make_share,
                     topk_gap, zipf_targets)
