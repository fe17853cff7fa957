"""CPU oracle for the batched GQA decode step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy (float64) statement of what one decode
iteration computes.  Only the test suite, the smoke check and the benchmark's
``cpu_baseline`` leg may import it.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product path: the two share only the seeded input generators.

Pins (checked by the CPU tests against things other than this code):
  * ``kvcache``: block allocator and slot map -- brute-force invariants and an
    expansion of the block table into a flat slot list.
  * ``decoder``: bf16 rounding (against torch's conversion), RMSNorm (against
    ``torch.nn.functional.rms_norm`` and a closed form), RoPE (identity at
    position 0, pair norms, relative-position property, and the LLaMA rotary
    routine of ``transformers``), attention (single cached token returns V,
    constant V, softmax rows sum to one, torch SDPA with GQA on a dense copy),
    the whole layer and the whole step (``transformers`` LLaMA decoder with a
    supplied KV cache), and the nano-batch split (equal to the unsplit step).
"""
