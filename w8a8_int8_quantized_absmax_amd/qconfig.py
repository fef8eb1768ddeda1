"""The PDMIX quantization config of the configuration workflow guide, validated.

[PDMIX-guide] section 4, step 2 (the recommended config: a `linear_quant`
processor with `qconfig.act` and `qconfig.weight`, each with scope, dtype,
symmetric and method) and step 3 (the configuration item table): the four
activation fields are fixed by the algorithm -- scope pd_mix (prefill per
token, decode per tensor), int8, symmetric false (the registered decode
scheme is asymmetric), the MinMax observer -- and the weight fields are the
companion combination that this library's weight quantizer implements:
per-channel, int8, symmetric, MinMax (absmax).  There is nothing to tune: a
config that asks for anything else is refused, naming the field, and a valid
one maps onto the library calls that realise it.

The config is read from a mapping (for instance `yaml.safe_load` of the
guide's YAML); nothing here touches the GPU.
"""
from __future__ import annotations

import dataclasses

# the activation fields the algorithm fixes ([PDMIX-guide] step 3)
FIXED_ACT = {"scope": "pd_mix", "dtype": "int8", "symmetric": False, "method": "minmax"}
# the weight combination this library implements (pdq_quantize_weight)
SUPPORTED_WEIGHT = {"scope": "per_channel", "dtype": "int8", "symmetric": True, "method": "minmax"}


class QConfigError(ValueError):
    """A config field this implementation of PDMIX cannot honour."""


@dataclasses.dataclass(frozen=True)
class PDMixConfig:
    """One validated `linear_quant` qconfig and the library calls that realise it."""

    act: tuple = tuple(sorted(FIXED_ACT.items()))
    weight: tuple = tuple(sorted(SUPPORTED_WEIGHT.items()))

    # which entry point runs each part of the method
    weight_quantization: str = "pdq_quantize_weight"  # offline, once: per-channel symmetric INT8 + code sums
    calibration: str = "pdq_calibrate_static"  # offline: MinMax over the calibration batches -> per-tensor S, Z
    prefill: str = "pdq_linear_prefill"  # per-token dynamic symmetric activations
    decode: str = "pdq_linear_decode"  # per-tensor static asymmetric activations (the calibrated S, Z)


def _check_section(name: str, got, want: dict) -> None:
    if not isinstance(got, dict):
        raise QConfigError(f"qconfig.{name} must be a mapping, got {type(got).__name__}")
    unknown = sorted(set(got) - set(want))
    if unknown:
        raise QConfigError(f"qconfig.{name}: unknown field(s) {unknown}")
    missing = sorted(set(want) - set(got))
    if missing:
        raise QConfigError(f"qconfig.{name}: missing field(s) {missing}")
    for key, value in want.items():
        v = got[key]
        same = (v is value) if isinstance(value, bool) else (isinstance(v, str) and v.lower() == value)
        if not same:
            if name == "act":
                why = "fixed by the PDMIX algorithm"
            else:
                why = "the weight quantizer here is per-channel symmetric INT8 MinMax"
            raise QConfigError(f"qconfig.{name}.{key} = {v!r}: only {value!r} is supported ({why})")


def parse_qconfig(qconfig: dict) -> PDMixConfig:
    """Validate one `qconfig` mapping (its `act` and `weight` sections)."""
    if not isinstance(qconfig, dict):
        raise QConfigError(f"qconfig must be a mapping, got {type(qconfig).__name__}")
    unknown = sorted(set(qconfig) - {"act", "weight"})
    if unknown:
        raise QConfigError(f"qconfig: unknown section(s) {unknown}")
    for section, want in (("act", FIXED_ACT), ("weight", SUPPORTED_WEIGHT)):
        if section not in qconfig:
            raise QConfigError(f"qconfig: missing section {section!r}")
        _check_section(section, qconfig[section], want)
    return PDMixConfig()


def parse_spec(spec: dict) -> list[PDMixConfig]:
    """Validate every `linear_quant` processor of a `spec` mapping (the guide's
    top-level key, or the mapping under it); other processor types are not
    this library's and are refused."""
    if isinstance(spec, dict) and "spec" in spec:
        spec = spec["spec"]
    if not isinstance(spec, dict) or not isinstance(spec.get("process"), list) or not spec["process"]:
        raise QConfigError("spec.process must be a non-empty list of processors")
    out = []
    for i, proc in enumerate(spec["process"]):
        if not isinstance(proc, dict):
            raise QConfigError(f"spec.process[{i}] must be a mapping")
        if proc.get("type") != "linear_quant":
            raise QConfigError(f"spec.process[{i}].type = {proc.get('type')!r}: only 'linear_quant' is supported")
        if "qconfig" not in proc:
            raise QConfigError(f"spec.process[{i}]: missing qconfig")
        out.append(parse_qconfig(proc["qconfig"]))
    return out
