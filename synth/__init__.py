"""Seeded synthetic inputs for the confidence-scheduled ragged verify path.

This package only draws inputs. It computes none of the method's steps: no
confidence head, no survival product, no cut, no packing, no argmax and no
acceptance. Both the oracle (under ``oracle/``) and the HIP path receive the
arrays it returns; neither side imports the other.
"""
from .configs import CONFIGS, Config, config_by_name
from .gen import (StepInputs, bf16_bits_from_f32, bf16_bits_to_f32, make_params,
                  make_step, rne_bf16)

__all__ = ["CONFIGS", "Config", "config_by_name", "StepInputs", "bf16_bits_from_f32",
           "bf16_bits_to_f32", "make_params", "make_step", "rne_bf16"]
