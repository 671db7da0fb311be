"""Seeded synthetic inputs (no method arithmetic); see synth.py and workloads.py."""
