"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package only draws inputs: Gaussian parameters, cameras and upstream
pixel gradients. It holds none of the rasterizer's arithmetic. Every array
is float32, structure-of-arrays, in the layouts the C-ABI takes.
"""
from .scenes import (CONFIGS, config_scene, look_at_camera, random_scene, shell_scene,
                     upstream_gradient, view_camera)

__all__ = ["CONFIGS", "config_scene", "look_at_camera", "random_scene", "shell_scene",
           "upstream_gradient", "view_camera"]
