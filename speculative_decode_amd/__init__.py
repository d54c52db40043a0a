"""MI355X-native fused Gated DeltaNet speculative-decode state update.

``ops`` holds the binding to the HIP library (loaded on first use; calls fail
loudly if it is not built), ``workloads`` the seeded synthetic inputs.
"""
__all__ = ["ops", "workloads"]
