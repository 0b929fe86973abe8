"""Oracle for the page-table-aware fused MoE layer and its page allocator.

TEST INFRASTRUCTURE ONLY. Plain, slow CPU code (numpy, fp64) written from
the Rimuru pages: the paper summary's abstract and Table 1, Figures 6-7
(multi-view layout, multi-level allocation), and the explainer's paragraphs
on moving the fence and on the page-table-aware kernel. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
never does, and this package imports nothing from the product.

Parity status of each function is stated in its module header.
"""
