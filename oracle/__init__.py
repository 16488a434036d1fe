"""CPU oracle of the GPT-2 training step (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
package.  See gpt2_oracle.c for what it computes and oracle.py for the wrapper.
"""
