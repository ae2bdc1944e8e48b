"""The CPU oracle of the MoE expert-FFN layer.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``. The library (``expert_ffn_layer_amd``) never imports, links or runs it.
"""
