"""CPU oracle for the TTT-E2E inner loop and the E2-TTT chunk-end state.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the bench's
CPU-baseline leg may import anything from this package; the product path
never does. It shares no code with the HIP library: it is plain NumPy (and,
in ``autograd_ref``, plain PyTorch CPU autograd) written from the method's
pages, in float64 for the fp32 workloads and float32 on bf16-valued inputs
for the bf16 workloads.

Modules
  ttt_e2e      -- model forward, hand-derived backward, mini-batch TTT loop,
                  plain (no-TTT) forward, decode continuation.
  autograd_ref -- an independent re-implementation of the loop in torch with
                  autograd gradients; it pins the hand-derived backward.
  e2ttt        -- E2-TTT per-token recursion and its closed-form chunk end.

Every function is pinned by a `-m "not gpu"` test (tests/test_oracle_*.py).
Parity unpinned against the pages (readings only; see the design notes):
the key/value store semantics across mini-batches, the MEAN/SUM reduction
choice, the static-then-dynamic wiring of the dual MLP and the tied lm_head.
These are pinned oracle-to-GPU only.
"""
