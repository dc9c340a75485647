"""CPU oracle of the MoE layer forward pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the product library never imports, links or calls it.
"""
