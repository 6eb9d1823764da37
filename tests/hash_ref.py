"""SplitMix64 counter-hash uniforms with Python integers, written from the
published definition (Steele, Lea and Flood, OOPSLA 2014; Vigna's splitmix64):
a reference for the tests that shares nothing with the oracle or the library."""
M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def mix(x):
    # the output function, reduced mod 2^64 after every step
    z = (x + GOLDEN) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def key(seed, row, pos, purpose):
    return mix(mix(mix(mix(seed & M64) ^ (row & M64)) ^ (pos & M64)) ^ (purpose & M64))


def uniform_bits(seed, row, pos, purpose):
    """The uniform as the integer k in k * 2^-53 (its top 53 bits)."""
    return key(seed, row, pos, purpose) >> 11
