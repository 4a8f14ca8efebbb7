"""Build the oracle's shared library: ``python -m oracle.build``."""
from oracle import build_library

if __name__ == "__main__":
    print(build_library())
