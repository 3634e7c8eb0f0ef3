"""CPU fp64 oracle for Hierarchical Global Attention (HGA) routed exact-token
attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The HIP product path never imports it, and this package imports
nothing from the HIP path; the two share only the seeded input generators in
``workloads``.

* ``hga_ref``  -- vectorised NumPy float64 implementation of every step.
* ``brute``    -- pure-Python loops over tokens, pairs and keys, for tiny inputs.

Sources (pages on arXiv:2606.30709, "Hierarchical Global Attention"):
the xllm-io paper-review page, section 3 (technical architecture): the
framework paragraph (chunks of C tokens split into groups of g_s), Eq. (1)
(dense causal attention), Eq. (2) (token-attention cost), the Mixed-RoPE
summary equation, the routing-policy rules and the top-K_c / top-K_g
selection equation, and the exact-token output paragraph; Sec. 5.5 as given
there (RoPE position index wrapped modulo 65536, the ``period`` option of
``hga_ref.rope_position``); the gradients of exact-token attention over fixed
routes (``hga_ref.attend_backward``, the training path the pages time);
RoPE itself follows RoFormer (cited by the pages).

Readings where the pages are silent are listed in each function's docstring.
Parity unpinned (conventions with no page value behind them, checked only as
oracle-vs-GPU under the stated reading): the half-split RoPE pair layout, the
fractional middle position beyond the closed-form consistency check, the
strict "<" of the wavelength split and the max aggregation of scores over the
query chunk x GQA group.
"""
