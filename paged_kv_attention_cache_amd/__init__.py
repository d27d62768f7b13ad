"""Paged KV write and paged attention for MI355X (placeholder until the binding lands)."""
