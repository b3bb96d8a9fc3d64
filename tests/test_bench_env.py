"""bench.py's runtime setting (CPU): kernel arguments in device memory unless
the environment already chooses, set before torch is imported, and reported
as the line's runtime_env."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env_after_import(extra):
    env = {k: v for k, v in os.environ.items() if k != "HIP_FORCE_DEV_KERNARG"}
    env.update(extra)
    code = ("import sys, os; sys.path.insert(0, %r); import bench; "
            "print(os.environ.get('HIP_FORCE_DEV_KERNARG')); print('torch' in sys.modules)" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
    return out.stdout.split()


def test_default_is_device_kernel_arguments_before_torch():
    value, torch_loaded = _env_after_import({})
    assert value == "1"
    assert torch_loaded == "False"   # set before the HIP runtime can initialise


def test_explicit_setting_is_kept():
    value, _ = _env_after_import({"HIP_FORCE_DEV_KERNARG": "0"})
    assert value == "0"


def test_record_reports_the_setting():
    code = ("import sys; sys.path.insert(0, %r); import bench, types; "
            "a = types.SimpleNamespace(steps=1, warmup=0); "
            "print(bench.base_record(a, 'm', 1.0, 1.0, 'w')['runtime_env']['HIP_FORCE_DEV_KERNARG'])" % ROOT)
    env = {k: v for k, v in os.environ.items() if k != "HIP_FORCE_DEV_KERNARG"}
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "1"
